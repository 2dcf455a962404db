// Instantiated configurations of the skinny kernel, one X(...) per variant,
// in variant order: X(MB, WK, U, CP, AL)
//   MB   16-row blocks of A covered (the variant takes M <= 16 MB)
//   WK   waves per workgroup, splitting the workgroup's K range
//   U    32-k steps per chunk of loads (two chunks in flight per wave)
//   CP   cache-policy bits of the streamed B loads (0 default, 2 non-temporal)
//   AL   1: A fragments staged through LDS by full-line copies; 0: loaded directly
// The first variant with a given MB is the planner's default for that M.
// The build script reads this list to map code objects to variants.
#pragma once

#define HKG_SKINNY_CONFIGS(X) \
    X(1, 8, 8, 0, 0)          \
    X(2, 8, 4, 0, 0)          \
    X(4, 8, 2, 0, 0)          \
    X(8, 8, 2, 0, 0)          \
    X(1, 8, 8, 0, 1)          \
    X(2, 8, 4, 0, 1)          \
    X(1, 8, 4, 0, 1)
