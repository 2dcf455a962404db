// Instantiated configurations of the skinny kernel, one X(...) per variant,
// in variant order: X(MB, NB, WK, U, CP, AL)
//   MB   16-row blocks of A covered (the variant takes M <= 16 MB)
//   NB   16-row blocks of B (16 NB columns of C) per workgroup
//   WK   waves per workgroup, splitting the workgroup's K range
//   U    32-k steps per chunk of loads (two chunks in flight per wave)
//   CP   cache-policy bits of the streamed B loads (0 default, 2 non-temporal)
//   AL   1: A staged through LDS by 1 KB copies (MB <= 2); 0: A fragments
//        loaded straight into registers
// The build script reads this list to map code objects to variants.
#pragma once

#define HKG_SKINNY_CONFIGS(X) \
    X(1, 1, 8, 8, 0, 0)       \
    X(2, 1, 8, 4, 0, 0)       \
    X(4, 1, 8, 2, 0, 0)       \
    X(8, 1, 8, 2, 0, 0)       \
    X(1, 2, 8, 4, 0, 0)       \
    X(1, 4, 8, 4, 0, 0)       \
    X(1, 8, 8, 2, 0, 0)       \
    X(2, 4, 8, 2, 0, 0)       \
    X(4, 2, 8, 2, 0, 0)       \
    X(8, 2, 8, 1, 0, 0)       \
    X(1, 1, 8, 4, 0, 1)

// MXFP8 instantiations, same fields; U counts steps of 128 k.
#define HKG_MX_SKINNY_CONFIGS(X) \
    X(1, 1, 8, 4, 0, 0)          \
    X(2, 1, 8, 2, 0, 0)          \
    X(1, 1, 8, 4, 0, 1)          \
    X(2, 1, 8, 2, 0, 1)

// MXFP4 instantiations, same fields; U counts steps of 256 k (128 bytes of a
// row, two 128-k scaled MFMA halves).
#define HKG_MX4_SKINNY_CONFIGS(X) \
    X(1, 1, 8, 2, 0, 1)           \
    X(2, 1, 8, 2, 0, 1)           \
    X(2, 2, 8, 1, 0, 1)           \
    X(2, 4, 8, 1, 0, 1)
