// rssm_dispatch.h -- switch from runtime sizes/formats to kernel template
// arguments (key dim 16..256, input dtype, read-copy format).  RSSM_DISPATCH_RC
// sits inside RSSM_DISPATCH_N (it needs NN): MXFP4 blocks are 32 entries, so
// key dims below 32 have no MXFP4 kernels.
#pragma once

#define RSSM_DISPATCH_N(N_, ...)                                      \
    switch (N_) {                                                     \
        case 16: { constexpr int NN = 16; __VA_ARGS__; } break;       \
        case 32: { constexpr int NN = 32; __VA_ARGS__; } break;       \
        case 64: { constexpr int NN = 64; __VA_ARGS__; } break;       \
        case 128: { constexpr int NN = 128; __VA_ARGS__; } break;     \
        case 256: { constexpr int NN = 256; __VA_ARGS__; } break;     \
        default: return hipErrorInvalidValue;                         \
    }
#define RSSM_DISPATCH_IN(I_, ...)                                     \
    switch (I_) {                                                     \
        case IN_F32: { constexpr int II = IN_F32; __VA_ARGS__; } break;   \
        case IN_BF16: { constexpr int II = IN_BF16; __VA_ARGS__; } break; \
        default: return hipErrorInvalidValue;                         \
    }
#define RSSM_DISPATCH_RC(R_, ...)                                     \
    switch (R_) {                                                     \
        case RC_NONE: { constexpr int RCC = RC_NONE; __VA_ARGS__; } break; \
        case RC_BF16: { constexpr int RCC = RC_BF16; __VA_ARGS__; } break; \
        case RC_FP8: { constexpr int RCC = RC_FP8; __VA_ARGS__; } break;   \
        case RC_MXFP4: {                                              \
            if (NN < 32) return hipErrorInvalidValue;                 \
            constexpr int RCC = NN < 32 ? RC_NONE : RC_MXFP4;         \
            __VA_ARGS__;                                              \
        } break;                                                      \
        default: return hipErrorInvalidValue;                         \
    }
// The same without MXFP4 (kernels that keep 32 q values per query per lane
// in registers, and the reset kernel, which has no key-dim template).
#define RSSM_DISPATCH_RC3(R_, ...)                                    \
    switch (R_) {                                                     \
        case RC_NONE: { constexpr int RCC = RC_NONE; __VA_ARGS__; } break; \
        case RC_BF16: { constexpr int RCC = RC_BF16; __VA_ARGS__; } break; \
        case RC_FP8: { constexpr int RCC = RC_FP8; __VA_ARGS__; } break;   \
        default: return hipErrorInvalidValue;                         \
    }

// Checkpoint storage format (CK_F32, CK_F16 or CK_FP8).
#define RSSM_DISPATCH_CK(C_, ...)                                     \
    switch (C_) {                                                     \
        case CK_F32: { constexpr int CKK = CK_F32; __VA_ARGS__; } break;  \
        case CK_F16: { constexpr int CKK = CK_F16; __VA_ARGS__; } break;  \
        case CK_FP8: { constexpr int CKK = CK_FP8; __VA_ARGS__; } break;  \
        default: return hipErrorInvalidValue;                         \
    }
// The same inside RSSM_DISPATCH_RC: an fp8 checkpoint is only used with a
// read copy, so the pair (RC_NONE, CK_FP8) has no kernels.
#define RSSM_DISPATCH_CK_RC(C_, ...)                                  \
    switch (C_) {                                                     \
        case CK_F32: { constexpr int CKK = CK_F32; __VA_ARGS__; } break;  \
        case CK_F16: { constexpr int CKK = CK_F16; __VA_ARGS__; } break;  \
        case CK_FP8: {                                                \
            if (RCC == RC_NONE) return hipErrorInvalidValue;          \
            constexpr int CKK = RCC == RC_NONE ? CK_F32 : CK_FP8;     \
            __VA_ARGS__;                                              \
        } break;                                                      \
        default: return hipErrorInvalidValue;                         \
    }
// Read formats of verification (a copy, or the checkpoint itself).
#define RSSM_DISPATCH_RD(R_, ...)                                     \
    switch (R_) {                                                     \
        case RC_F16: { constexpr int RCC = RC_F16; __VA_ARGS__; } break;   \
        default: RSSM_DISPATCH_RC(R_, __VA_ARGS__);                   \
    }
#define RSSM_DISPATCH_RD3(R_, ...)                                    \
    switch (R_) {                                                     \
        case RC_F16: { constexpr int RCC = RC_F16; __VA_ARGS__; } break;   \
        default: RSSM_DISPATCH_RC3(R_, __VA_ARGS__);                  \
    }
