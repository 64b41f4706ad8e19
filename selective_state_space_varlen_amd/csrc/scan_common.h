// Shared layout of the selective-scan workspace and tiling constants.
#pragma once

#include "common.h"

namespace ssmp {

// Time tiling. A chunk of kLC tokens is the unit of time parallelism: one
// wave walks it serially for 64 channels, and chunks are joined by the affine
// carry h_out = P h_in + S (P = 0 once the chunk holds a head). The forward
// also stores the state every kCK tokens; the backward restarts from those
// and replays kK-token sub-chunks with their states held in registers.
constexpr int kLC = 256;
constexpr int kCK = 16;
constexpr int kK = 4;
static_assert(kLC % kCK == 0 && kCK % kK == 0, "tiling");

struct ScanWs {
    int64_t nck;      // checkpoint slots: slot j holds the state entering token j*kCK
    int64_t nchunk;   // chunks of kLC tokens
    int64_t ngroup;   // channel groups of 64
    // offsets in floats from the workspace base
    size_t ckpt;      // [nck][N][D]
    size_t P, S;      // [nchunk][N][D]   forward: chunk decay and local end state
    size_t Pr, Sr;    // [nchunk][N][D]   backward: reverse-carry summaries
    size_t cin;       // [nchunk][N][D]   backward: carry entering each chunk from the right
    size_t dApart;    // [nchunk][N][D]
    size_t dDpart;    // [nchunk][D]
    size_t dBC;       // [ngroup][T][2N]
    size_t total;     // floats
};

inline ScanWs scan_ws_layout(int64_t T, int D, int N) {
    ScanWs w{};
    w.nck = (T + kCK - 1) / kCK;
    w.nchunk = (T + kLC - 1) / kLC;
    w.ngroup = (D + kWave - 1) / kWave;
    const size_t ND = (size_t)N * D;
    size_t off = 0;
    w.ckpt = off; off += (size_t)w.nck * ND;
    const size_t scratch = off;
    // forward scratch
    w.P = scratch; w.S = w.P + (size_t)w.nchunk * ND;
    const size_t fwd_end = w.S + (size_t)w.nchunk * ND;
    // backward scratch (reuses the same region)
    w.Pr = scratch; w.Sr = w.Pr + (size_t)w.nchunk * ND;
    w.cin = w.Sr + (size_t)w.nchunk * ND;
    w.dApart = w.cin + (size_t)w.nchunk * ND;
    w.dDpart = w.dApart + (size_t)w.nchunk * ND;
    w.dBC = w.dDpart + (size_t)w.nchunk * D;
    const size_t bwd_end = w.dBC + (size_t)w.ngroup * (size_t)T * 2 * N;
    w.total = fwd_end > bwd_end ? fwd_end : bwd_end;
    return w;
}

// Flat 1-D grid over (chunk, 64-channel group), group fastest: concurrently
// running waves cover adjacent channels of the same tokens.
struct Tile {
    int g;      // channel group
    int64_t c;  // chunk
};
__device__ __forceinline__ Tile tile_of(int D) {
    const unsigned ng = (unsigned)((D + kWave - 1) / kWave);
    return Tile{(int)(blockIdx.x % ng), (int64_t)(blockIdx.x / ng)};
}

inline int scan_check_args(int64_t T, int D, int N, int dtype) {
    if (T < 0 || D < 1) return SSMP_ERR_SHAPE;
    if (T >= (int64_t(1) << 31)) return SSMP_ERR_SHAPE;
    if (((T + kLC - 1) / kLC) * ((D + kWave - 1) / kWave) >= (int64_t(1) << 31)) return SSMP_ERR_SHAPE;
    if ((T * (int64_t)D) >= (int64_t(1) << 40)) return SSMP_ERR_SHAPE;
    if (!(N == 1 || N == 2 || N == 4 || N == 8 || N == 16)) return SSMP_ERR_UNSUPPORTED;
    if (dtype != SSMP_F32 && dtype != SSMP_BF16) return SSMP_ERR_UNSUPPORTED;
    return SSMP_OK;
}

}  // namespace ssmp
