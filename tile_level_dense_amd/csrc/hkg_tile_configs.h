// Instantiated configurations of the tile kernel, one X(...) per variant,
// in variant order: X(BM, BN, BK, STAGES, WM, WN, SCHED)
//   BM x BN   output tile of one workgroup
//   BK        k per LDS stage (32 or 64)
//   STAGES    LDS stages in the ring (prefetch distance STAGES - 1)
//   WM x WN   wave grid (WM * WN waves; each wave owns BM/WM x BN/WN of C)
//   SCHED     0: compiler-scheduled fragment reads; 1: reads of the next
//             32-k step interleaved with the MFMAs of the current one;
//             2: fragment reads of the next 32-k step (also across stages)
//             overlap the current MFMAs; branch-free ring with STAGES - 1
//             copies ahead; 5: ping-pong of two 4-wave groups (256 x 256 x
//             64 tile, 8 waves; STAGES is not used), copies issued only in
//             memory phases, A halves double- and B triple-buffered; 6: the
//             same ping-pong on a persistent grid of one workgroup per CU,
//             each walking several tiles as one stream of stages (without a
//             fused epilogue; with one, it runs as 5); 7: k-interleaved
//             ping-pong, two groups of WM x WN waves, each group over the
//             whole tile, taking alternate 64-k stages (STAGES 3 or 5 in
//             LDS, copies 2 or 4 stages ahead; the partial tiles are added
//             through LDS; no split-K)
// The build script reads this list to map code objects to variants.
#pragma once

#define HKG_TILE_CONFIGS(X)       \
    X(256, 256, 64, 2, 4, 2, 5)   \
    X(256, 128, 64, 2, 4, 2, 2)   \
    X(128, 128, 64, 2, 2, 2, 2)   \
    X(128, 128, 64, 2, 2, 2, 0)   \
    X(256, 256, 64, 2, 2, 4, 2)   \
    X(256, 256, 64, 2, 2, 4, 5)   \
    X(256, 256, 64, 2, 2, 4, 0)   \
    X(64, 64, 64, 4, 2, 2, 2)     \
    X(128, 128, 64, 4, 2, 2, 2)   \
    X(64, 128, 64, 4, 2, 2, 2)    \
    X(128, 64, 64, 4, 2, 2, 2)     \
    X(256, 256, 64, 2, 4, 2, 6)    \
    X(64, 96, 64, 4, 2, 2, 2)      \
    X(128, 96, 64, 4, 2, 2, 2)     \
    X(128, 256, 64, 3, 2, 2, 7)    \
    X(128, 128, 64, 3, 2, 2, 7)    \
    X(128, 128, 64, 5, 2, 2, 7)

// MXFP8 instantiations (E4M3 operands, E8M0 scale per 32 k), same fields;
// BK = 128 k (128 bytes per row, as the bf16 BK = 64), SCHED 5 or 0 (a
// two-stage ring).  Wave tiles are whole 64-row scale groups.
#define HKG_MX_TILE_CONFIGS(X)     \
    X(256, 256, 128, 2, 4, 2, 5)   \
    X(128, 128, 128, 2, 2, 2, 0)

// MXFP4 instantiations (E2M1 operands two per byte, E8M0 scale per 32 k),
// same fields; BK = 256 k (again 128 bytes per row: two 128-k scaled MFMA
// steps per stage), SCHED 5 or 0 as for MXFP8.
#define HKG_MX4_TILE_CONFIGS(X)    \
    X(256, 256, 256, 2, 4, 2, 5)   \
    X(128, 128, 256, 2, 2, 2, 0)

// Grouped (mixture-of-experts) instantiations on a persistent grid, same
// fields; bf16 only, K split only in a partial last round.  Variant 3 (the
// ping-pong whose workgroups stream their tiles' stages; with a fused
// epilogue it runs as 2) and 1 are the planner's; 0 (register-pipelined) and
// 2 (the ping-pong one tile at a time) are kept as alternatives.
#define HKG_GROUPED_CONFIGS(X)     \
    X(256, 256, 64, 2, 2, 4, 2)    \
    X(128, 128, 64, 2, 2, 2, 2)    \
    X(256, 256, 64, 2, 4, 2, 5)    \
    X(256, 256, 64, 2, 4, 2, 6)
