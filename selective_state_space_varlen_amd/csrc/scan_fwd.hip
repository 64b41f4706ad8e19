// selective_scan_pack forward.
//
// Shanghai AI Lab article on packed variable-length Mamba-1 training
// (gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), sections "SSM_pack算子" and
// "基本原理": the state crosses packed sequences only through the recurrence,
// so it is reset to zero at every head token. Per channel d, state n:
//   h_t = exp(delta_t A[d,n]) h_{t-1} + delta_t B_t[n] u_t   (h_{t-1} = 0 at heads)
//   y_t = sum_n C_t[n] h_t[n] + Dskip[d] u_t,   out_t = y_t SiLU(z_t)
//
// Mapping: one lane per channel, the d_state values in VGPRs, one wave per
// (chunk of lc tokens, 64 channels). B_t and C_t are the same for the whole
// wave: an fp32 copy made first arrives through scalar loads. Per-lane inputs
// are staged through LDS in kFwdBlock-token blocks, the next block in flight
// while the current one is computed. The time axis is joined across chunks by the
// article's reset rule applied to the affine carry (h_out = P h_in + S, with
// the multiplier P zeroed once a head is passed):
//   1. summary: per chunk, from its last head (or its start) to its end,
//      S = end state from zero and P = product of decays (0 if a head was
//      seen). P[n] = exp2(A2[n] sum delta) is kept as the channel's sum of
//      delta (NaN for 0), N times fewer bytes. Skipped when the next chunk
//      starts with a head.
//   2. carry: per (n, d), a sequential pass over chunks gives the state
//      entering each chunk.
//   3. output: each chunk replays its tokens from that state, writes out and,
//      when the caller keeps checkpoints for the backward, stores the state
//      entering every ci-th token.
// A fourth kernel, used by the backward, replays the recurrence without the
// output from kept states to the dense checkpoints the backward restarts from.
// The step map and gate floor (ScanOpts) apply where delta and z are read;
// carried sequence states enter at heads and leave at ends, in the blocks
// that already take the slow path for heads.
#include "scan_common.h"

#include <mutex>

namespace ssmp {

constexpr int kFwdBlock = 8;  // tokens per staged block in the forward kernels
static_assert(kFwdBlock % kCK == 0, "a block holds whole checkpoint intervals");

// B (and C) rows of BT tokens from the fp32 copy, prefetched one token ahead
// so the scalar loads of token k+1 overlap the arithmetic of token k.
template <int NROW>
__device__ __forceinline__ void load_rowv(const float* __restrict__ p, float (&v)[NROW]) {
#pragma unroll
    for (int j = 0; j < NROW; ++j) v[j] = p[j];
}

// Summary recurrence over one block: h = a h + dtu B from zero state. SAFE
// blocks skip tokens before `first` or past `nt`; fast blocks hold neither.
template <bool SAFE, typename T, int NS, int BT, typename St>
__device__ __forceinline__ void summary_block(const T* lds, const float* __restrict__ bc, int64_t tb, int first,
                                              int nt, const float (&A2)[NS], float (&h)[NS], float& sdt, float& cdt,
                                              int lane, const StepMap& sm) {
    // the block's per-lane inputs are read from LDS before the first scalar
    // load: a wait for LDS data also waits for scalar loads in flight
    float dtv[BT], uv[BT];
#pragma unroll
    for (int k = 0; k < BT; ++k) {
        dtv[k] = St::get(lds, 1, k, lane);
        uv[k] = St::get(lds, 0, k, lane);
    }
    if (sm.on) {
#pragma unroll
        for (int k = 0; k < BT; ++k) dtv[k] = sm.eff(dtv[k]);
    }
    const float* __restrict__ rows = bc + (size_t)tb * 2 * NS;
    float cur[NS];
    load_rowv<NS>(rows + (SAFE ? first : 0) * 2 * NS, cur);
#pragma unroll
    for (int k = 0; k < BT; ++k) {
        if constexpr (SAFE) {
            if (k < first) continue;
            if (k >= nt) break;
        }
        float nxt[NS];
        const bool more = SAFE ? (k + 1 < nt) : (k + 1 < BT);
        scalar_loads_done();
        if (more) load_rowv<NS>(rows + (k + 1) * 2 * NS, nxt);
        __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of this token's arithmetic
        const float dt = dtv[k];
        const float dtu = dt * uv[k];
        // compensated sum of delta: the chunk's decay is exp2(A2 * sum delta)
        const float yk = dt - cdt;
        const float tk = sdt + yk;
        cdt = (tk - sdt) - yk;
        sdt = tk;
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = __builtin_fmaf(exp2_fast(dt * A2[n]), h[n], dtu * cur[n]);
        if (more) {
#pragma unroll
            for (int n = 0; n < NS; ++n) cur[n] = nxt[n];
        }
    }
}

template <typename T, int NS>
__global__ __launch_bounds__(64, 4) void k_scan_fwd_summary(const T* __restrict__ u, const T* __restrict__ delta,
                                                         const float* __restrict__ A, const float* __restrict__ bc,
                                                         const int32_t* __restrict__ pos, float* __restrict__ P,
                                                         float* __restrict__ S, int64_t T_, int D, int vec, int lc,
                                                         ScanOpts opt) {
    constexpr int BT = kFwdBlock;
    using St = Stager<T, 2, BT>;
    __shared__ __attribute__((aligned(16))) T lds[St::kElems];
    const int lane = threadIdx.x;
    const Tile tl = tile_of(D);
    const int d = tl.g * kWave + lane;
    const bool act = d < D;
    const int dd = act ? d : D - 1;
    const int64_t c = tl.c;
    const int64_t t0 = c * lc;
    const int64_t t1 = (t0 + lc < T_) ? t0 + lc : T_;
    if (t1 >= T_) return;          // last chunk: no successor needs it
    if (pos[t1] == 0) return;      // successor starts at a head: its carry is zero

    // last head in [t0, t1): the summary starts there from a zero state
    int64_t ts = t0;
    bool has_head = false;
    for (int64_t base = t0; base < t1; base += kWave) {
        const int64_t t = base + lane;
        const bool f = (t < t1) && pos[t] == 0;
        const uint64_t m = __ballot(f);
        if (m) {
            has_head = true;
            ts = base + 63 - __builtin_clzll(m);
        }
    }
    float A2[NS], h[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        A2[n] = A[(size_t)dd * NS + n] * kLog2e;
        h[n] = 0.0f;
    }
    if (has_head && opt.h0) {
        // from the last head on, the state starts at that sequence's initial state
        const float* __restrict__ hp = opt.h0 + ((size_t)seq_of(opt.cu, opt.nseq, ts) * D + dd) * NS;
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = hp[n];
    }
    const StepMap sm = step_map(opt, dd);
    float sdt = 0.0f, cdt = 0.0f;
    const T* const src[2] = {u, delta};
    St st;
    const int64_t tb0 = t0 + ((ts - t0) / BT) * BT;
    st.fetch(src, tb0, T_, D, tl.g, lane, vec);
    for (int64_t tb = tb0; tb < t1; tb += BT) {
        wave_sync();
        st.commit(lds, src, tb, T_, D, tl.g, lane, vec);
        wave_sync();
        if (tb + BT < t1) st.fetch(src, tb + BT, T_, D, tl.g, lane, vec);
        const int first = (int)((ts > tb) ? ts - tb : 0);
        const int nt = (int)((tb + BT < t1) ? BT : t1 - tb);
        if (first == 0 && nt == BT)
            summary_block<false, T, NS, BT, St>(lds, bc, tb, 0, BT, A2, h, sdt, cdt, lane, sm);
        else
            summary_block<true, T, NS, BT, St>(lds, bc, tb, first, nt, A2, h, sdt, cdt, lane, sm);
    }
    if (act) {
        // the chunk's decay exp2(A2[n] * sdt) depends on n only through A: keep
        // sdt (NaN where a head cuts the chunk, i.e. decay 0) per channel
        P[(size_t)c * D + d] = has_head ? __builtin_nanf("") : sdt;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const size_t o = ((size_t)c * NS + n) * D + d;
            S[o] = h[n];
        }
    }
}

// State entering each chunk, in the checkpoint layout (hin[c]).
// P holds each chunk's sum of delta per channel (NaN: a head cuts the chunk).
template <int NS>
__global__ __launch_bounds__(256) void k_scan_fwd_carry(const float* __restrict__ P, const float* __restrict__ S,
                                                        const float* __restrict__ A,
                                                        const int32_t* __restrict__ pos, float* __restrict__ hin,
                                                        int64_t T_, int D, int64_t nchunk, int lc) {
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // n*D + d
    const int64_t ND = (int64_t)NS * D;
    const bool act = i0 < ND;
    const int64_t i = act ? i0 : ND - 1;  // lanes past the end run along (ballots need the wave) but store nothing
    // The summaries of kB chunks are loaded before the chain walks through
    // them, and the next kB are loaded while it does. Chunk c hands its state
    // on iff chunk c + 1 exists ((c + 1) lc < T); lane j < kB also loads the
    // position at the start of chunk cb + j + 1 (head test). Addresses step
    // by a fixed stride: the chain runs one wave per SIMD, so per-step index
    // arithmetic is not hidden by other waves.
    constexpr int kB = 16;
    const int lane = threadIdx.x % kWave;
    struct Batch {
        float P[kB], S[kB];
        int32_t hp;
    };
    const int dch = (int)(i % D);
    const float A2 = A[(size_t)dch * NS + (int)(i / D)] * kLog2e;
    auto load = [&](Batch& b, int64_t cb) {
        const int64_t tn = (cb + lane + 1) * lc;
        b.hp = (lane < kB && tn < T_) ? pos[tn] : 1;
        const float* p = P + (size_t)cb * D + dch;
        const float* q = S + (size_t)cb * ND + i;
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            if (cb + j + 1 < nchunk) {
                b.P[j] = *p;
                b.S[j] = *q;
            } else {
                b.P[j] = 0.0f;
                b.S[j] = 0.0f;
            }
            p += D;
            q += ND;
        }
    };
    float h = 0.0f;
    float* kp = hin + ck_index<NS>(dch, (int)(i / D), D);  // chunk c's entry state (checkpoint layout)
    const size_t kstride = (size_t)ND;
    Batch cur, nxt;
    load(cur, 0);
    for (int64_t cb = 0; cb < nchunk; cb += kB) {
        if (cb + kB < nchunk) load(nxt, cb + kB);
        const uint64_t heads = __ballot(cur.hp == 0);  // bit j: chunk cb + j + 1 starts at a head
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const int64_t c = cb + j;
            if (c < nchunk) {
                if (act) *kp = h;
                kp += kstride;
            }
            // decay 0 marks a chunk holding a head: select, so that a
            // non-finite state before the head cannot leak through 0 * h
            const float tj = cur.P[j];
            const float Pj = (tj != tj) ? 0.0f : exp2_fast(A2 * tj);
            const float hn = ((heads >> j) & 1u) ? 0.0f : (Pj == 0.0f) ? cur.S[j] : __builtin_fmaf(Pj, h, cur.S[j]);
            h = (c + 1 < nchunk) ? hn : h;
        }
        cur = nxt;
    }
}

// Output recurrence over one block of BT tokens. SAFE blocks may end early
// (nt < BT) and may hold heads; fast blocks are full and head-free, so their
// tokens run straight through with the next token's B/C rows in flight.
// With cish >= 0 the state entering every token t with t % 2^cish == 0 goes
// to checkpoint slot t >> cish of `saved`.
//
// With sequence states, a head starts from its sequence's initial state
// instead of zero, and the state after an end token (ends: bit k) is that
// sequence's final state; both occur only in SAFE blocks.
template <bool SAFE, bool GATE, bool XS, bool ST, typename T, int NS, int BT, typename St>
__device__ __forceinline__ void out_block(const T* lds, const float* __restrict__ bc, int64_t tb, int nt,
                                          uint32_t heads, uint32_t ends, const float (&A2)[NS], float (&h)[NS],
                                          float Dv, int lane, T* __restrict__ ob, int D, int d, int dd,
                                          float* __restrict__ saved, int cish, size_t ND, bool act,
                                          const StepMap& sm, const ScanOpts& opt) {
    const float gf = opt.gate_floor;
    // the block's per-lane inputs are read from LDS before the first scalar
    // load: a wait for LDS data also waits for scalar loads in flight
    float dtv[BT], uv[BT], zv[BT];
#pragma unroll
    for (int k = 0; k < BT; ++k) {
        dtv[k] = St::get(lds, 1, k, lane);
        uv[k] = St::get(lds, 0, k, lane);
        if constexpr (GATE) zv[k] = St::get(lds, 2, k, lane);
    }
    const float* __restrict__ rows = bc + (size_t)tb * 2 * NS;
    float cur[2 * NS];
    load_rowv<2 * NS>(rows, cur);
#pragma unroll
    for (int k = 0; k < BT; ++k) {
        if constexpr (SAFE) {
            if (k >= nt) break;
        }
        if (k % kMinCK == 0 && cish >= 0 && ((tb + k) & ((int64_t(1) << cish) - 1)) == 0)
            ck_store<NS>(saved + (size_t)((tb + k) >> cish) * ND, d, D, h);
        float nxt[2 * NS];
        const bool more = SAFE ? (k + 1 < nt) : (k + 1 < BT);
        scalar_loads_done();
        if (more) load_rowv<2 * NS>(rows + (k + 1) * 2 * NS, nxt);
        __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of this token's arithmetic
        // the step map next to its use: mapping the whole block first held
        // the first state update behind eight softplus chains
        const float dt = XS ? sm.eff(dtv[k]) : dtv[k];
        const float uu = uv[k];
        const float dtu = dt * uu;
        if constexpr (SAFE) {
            if ((heads >> k) & 1u) {
                asm volatile("");
                if (ST && opt.h0) {
                    const float* __restrict__ hp = opt.h0 + ((size_t)seq_of(opt.cu, opt.nseq, tb + k) * D + dd) * NS;
#pragma unroll
                    for (int n = 0; n < NS; ++n) h[n] = hp[n];
                } else {
#pragma unroll
                    for (int n = 0; n < NS; ++n) h[n] = 0.0f;
                }
            }
        }
        float y = 0.0f;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            h[n] = __builtin_fmaf(exp2_fast(dt * A2[n]), h[n], dtu * cur[n]);
            y = __builtin_fmaf(cur[NS + n], h[n], y);
        }
        if constexpr (SAFE && ST) {
            if (((ends >> k) & 1u) && act) {
                float* __restrict__ hq = opt.hT + ((size_t)seq_of(opt.cu, opt.nseq, tb + k) * D + d) * NS;
#pragma unroll
                for (int n = 0; n < NS; ++n) hq[n] = h[n];
            }
        }
        y = __builtin_fmaf(Dv, uu, y);
        if constexpr (GATE) {
            const float zz = zv[k];
            y *= __builtin_fmaf(zz, sigmoid_fast(zz), gf);
        }
        // the token's row as a buffer resource: a lane past D stores past its
        // end, which the hardware drops
        Elt<T>::template st_rsrc<kBufNT>(bytes_rsrc(ob + (size_t)k * D, (uint32_t)D * (uint32_t)sizeof(T)),
                                         (uint32_t)d * (uint32_t)sizeof(T), y);
        if (more) {
#pragma unroll
            for (int j = 0; j < 2 * NS; ++j) cur[j] = nxt[j];
        }
    }
}

// Four waves per SIMD (128 VGPRs) for the plain bf16 kernel. The state
// variant, whose heads load arbitrary states, the step-map variant, which
// holds the softplus temporaries, and fp32 inputs, whose staged block takes
// twice the registers, would spill at that budget in the hot loop; all of
// them run faster at up to 256 VGPRs (measured: 3 waves fit).
template <typename T, int NS, bool GATE, bool XS, bool ST>
__global__ __launch_bounds__(64, (ST || XS || sizeof(T) == 4) ? 2 : 4) void k_scan_fwd_out(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A, const float* __restrict__ bc,
    const float* __restrict__ Dskip, const T* __restrict__ z, const int32_t* __restrict__ pos, T* __restrict__ out,
    const float* __restrict__ hin, float* __restrict__ saved, int cish, int64_t T_, int D, int vec, int lc,
    ScanOpts opt) {
    constexpr int BT = kFwdBlock;
    using St = Stager<T, 3, BT>;
    __shared__ __attribute__((aligned(16))) T lds[St::kElems];
    const int lane = threadIdx.x;
    const Tile tl = tile_of(D);
    const int d = tl.g * kWave + lane;
    const bool act = d < D;
    const int dd = act ? d : D - 1;
    const int64_t c = tl.c;
    const int64_t t0 = c * lc;
    const int64_t t1 = (t0 + lc < T_) ? t0 + lc : T_;
    const size_t ND = (size_t)NS * D;

    float A2[NS], h[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        A2[n] = A[(size_t)dd * NS + n] * kLog2e;
        h[n] = 0.0f;
    }
    ck_load<NS, NS>(hin + (size_t)c * ND, dd, D, 0, act, h);
    const float Dv = (Dskip && act) ? Dskip[dd] : 0.0f;
    const StepMap sm = step_map(opt, dd);
    const T* const src[3] = {u, delta, GATE ? z : u};
    St st;
    st.fetch(src, t0, T_, D, tl.g, lane, vec);
    for (int64_t tb = t0; tb < t1; tb += BT) {
        const uint32_t heads = block_heads<BT>(pos, tb, T_, lane);
        const uint32_t ends = (ST && opt.hT) ? block_ends<BT>(pos, tb, T_, lane) : 0u;
        wave_sync();
        st.commit(lds, src, tb, T_, D, tl.g, lane, vec);
        wave_sync();
        if (tb + BT < t1) st.fetch(src, tb + BT, T_, D, tl.g, lane, vec);
        const int nt = (int)((tb + BT < t1) ? BT : t1 - tb);
        T* __restrict__ ob = out + (size_t)tb * D;
        if ((heads | ends) == 0 && nt == BT)
            out_block<false, GATE, XS, ST, T, NS, BT, St>(lds, bc, tb, BT, 0u, 0u, A2, h, Dv, lane, ob, D, d, dd,
                                                  saved, cish, ND, act, sm, opt);
        else
            out_block<true, GATE, XS, ST, T, NS, BT, St>(lds, bc, tb, nt, heads, ends, A2, h, Dv, lane, ob, D, d, dd,
                                                 saved, cish, ND, act, sm, opt);
    }
}

// Dense checkpoints: the output pass's recurrence without its output, from a
// kept state every G tokens, storing the state entering every kCK-th token.
// The arithmetic is the output pass's, operation for operation, so the
// replayed states equal the ones that pass would have kept.
template <bool SAFE, bool XS, bool ST, typename T, int NS, int BT, typename St>
__device__ __forceinline__ void replay_block(const T* lds, const float* __restrict__ bc, int64_t tb, int nt,
                                             uint32_t heads, const float (&A2)[NS], float (&h)[NS], int lane,
                                             float* __restrict__ ck, size_t ND, int d, int D, int dd, bool act,
                                             const StepMap& sm, const ScanOpts& opt) {
    float dtv[BT], uv[BT];
#pragma unroll
    for (int k = 0; k < BT; ++k) {
        dtv[k] = St::get(lds, 1, k, lane);
        uv[k] = St::get(lds, 0, k, lane);
    }
    const float* __restrict__ rows = bc + (size_t)tb * 2 * NS;  // B: the first NS of each row
    float cur[NS];
    load_rowv<NS>(rows, cur);
#pragma unroll
    for (int k = 0; k < BT; ++k) {
        if constexpr (SAFE) {
            if (k >= nt) break;
        }
        if (k % kCK == 0) ck_store<NS>(ck + (size_t)(k / kCK) * ND, d, D, h);
        float nxt[NS];
        const bool more = SAFE ? (k + 1 < nt) : (k + 1 < BT);
        scalar_loads_done();
        if (more) load_rowv<NS>(rows + (k + 1) * 2 * NS, nxt);
        __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of this token's arithmetic
        const float dt = XS ? sm.eff(dtv[k]) : dtv[k];
        const float dtu = dt * uv[k];
        if constexpr (SAFE) {
            if ((heads >> k) & 1u) {
                asm volatile("");
                if (ST && opt.h0) {
                    const float* __restrict__ hp = opt.h0 + ((size_t)seq_of(opt.cu, opt.nseq, tb + k) * D + dd) * NS;
#pragma unroll
                    for (int n = 0; n < NS; ++n) h[n] = hp[n];
                } else {
#pragma unroll
                    for (int n = 0; n < NS; ++n) h[n] = 0.0f;
                }
            }
        }
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = __builtin_fmaf(exp2_fast(dt * A2[n]), h[n], dtu * cur[n]);
        if (more) {
#pragma unroll
            for (int n = 0; n < NS; ++n) cur[n] = nxt[n];
        }
    }
}

// One wave per (segment of G tokens, 64 channels): segment c starts from
// start[c * sstride] (checkpoint layout) and writes dense slots t / kCK.
template <typename T, int NS, bool XS, bool ST>
__global__ __launch_bounds__(64, (ST || XS || sizeof(T) == 4) ? 2 : 4) void k_scan_fwd_replay(
    const T* __restrict__ u, const T* __restrict__ delta, const float* __restrict__ A, const float* __restrict__ bc,
    const int32_t* __restrict__ pos, const float* __restrict__ start, size_t sstride, float* __restrict__ dense,
    int64_t T_, int D, int vec, int G, ScanOpts opt) {
    constexpr int BT = kFwdBlock;
    using St = Stager<T, 2, BT>;
    __shared__ __attribute__((aligned(16))) T lds[St::kElems];
    const int lane = threadIdx.x;
    const Tile tl = tile_of(D);
    const int d = tl.g * kWave + lane;
    const bool act = d < D;
    const int dd = act ? d : D - 1;
    const int64_t c = tl.c;
    const int64_t t0 = c * G;
    const int64_t t1 = (t0 + G < T_) ? t0 + G : T_;
    const size_t ND = (size_t)NS * D;
    float A2[NS], h[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) A2[n] = A[(size_t)dd * NS + n] * kLog2e;
    ck_load<NS, NS>(start + (size_t)c * sstride, dd, D, 0, act, h);
    const StepMap sm = step_map(opt, dd);
    const T* const src[2] = {u, delta};
    St st;
    st.fetch(src, t0, T_, D, tl.g, lane, vec);
    for (int64_t tb = t0; tb < t1; tb += BT) {
        const uint32_t heads = block_heads<BT>(pos, tb, T_, lane);
        wave_sync();
        st.commit(lds, src, tb, T_, D, tl.g, lane, vec);
        wave_sync();
        if (tb + BT < t1) st.fetch(src, tb + BT, T_, D, tl.g, lane, vec);
        const int nt = (int)((tb + BT < t1) ? BT : t1 - tb);
        float* __restrict__ ck = dense + (size_t)(tb / kCK) * ND;
        if (heads == 0 && nt == BT)
            replay_block<false, XS, ST, T, NS, BT, St>(lds, bc, tb, BT, 0u, A2, h, lane, ck, ND, d, D, dd, act, sm,
                                                       opt);
        else
            replay_block<true, XS, ST, T, NS, BT, St>(lds, bc, tb, nt, heads, A2, h, lane, ck, ND, d, D, dd, act, sm,
                                                      opt);
    }
}

// Summary and carry passes: the state entering each chunk, at scratch + L.hin.
template <typename T, int NS>
static int scan_fwd_chunk_states(const void* u, const void* delta, const float* A, const int32_t* pos, float* ws,
                                 const ScanWs& L, int64_t T_, int D, const ScanOpts& opt, hipStream_t s) {
    const int lc = fwd_chunk_len(T_, D);
    const int64_t nchunk = L.nfchunk;
    const dim3 grid((unsigned)(L.ngroup * nchunk));
    const int vec = stage_vec_ok<T>(D, {u, delta}) ? 1 : 0;
    if (nchunk > 1) {
        k_scan_fwd_summary<T, NS><<<grid, kWave, 0, s>>>((const T*)u, (const T*)delta, A, ws + L.bc, pos, ws + L.P,
                                                         ws + L.S, T_, D, vec, lc, opt);
        SSMP_LAUNCH_CHECK();
    }
    const int64_t ND = (int64_t)NS * D;
    k_scan_fwd_carry<NS><<<(unsigned)((ND + 255) / 256), 256, 0, s>>>(ws + L.P, ws + L.S, A, pos, ws + L.hin, T_,
                                                                      D, nchunk, lc);
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

template <typename T, int NS>
static int scan_fwd_launch(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, const int32_t* pos, void* out, float* saved, int ci,
                           float* ws, int64_t T_, int D, const ScanOpts& opt, hipStream_t s) {
    const ScanWs L = scan_ws_layout(T_, D, NS, ci);
    const int lc = fwd_chunk_len(T_, D);
    const dim3 grid((unsigned)(L.ngroup * L.nfchunk));
    const int vec = stage_vec_ok<T>(D, {u, delta, z}) ? 1 : 0;
    k_bc_to_f32<T, NS><<<(unsigned)((T_ * 2 * NS + 255) / 256), 256, 0, s>>>((const T*)B, (const T*)C, ws + L.bc,
                                                                            T_);
    SSMP_LAUNCH_CHECK();
    int st = scan_fwd_chunk_states<T, NS>(u, delta, A, pos, ws, L, T_, D, opt, s);
    if (st) return st;
    const int cish = ci ? __builtin_ctz((unsigned)ci) : -1;
    const bool xs = opt.delta_bias != nullptr || opt.softplus != 0;
    // sequence states get kernels of their own, so the reset-only ones keep
    // their register allocation
    const bool sv = opt.h0 != nullptr || opt.hT != nullptr;
#define SSMP_FWD_OUT(G, X, S)                                                                                   \
    k_scan_fwd_out<T, NS, G, X, S><<<grid, kWave, 0, s>>>((const T*)u, (const T*)delta, A, ws + L.bc, Dskip,     \
                                                          G ? (const T*)z : nullptr, pos, (T*)out, ws + L.hin,    \
                                                          saved, cish, T_, D, vec, lc, opt)
#define SSMP_FWD_OUT_S(G, X)                \
    if (sv) SSMP_FWD_OUT(G, X, true);       \
    else SSMP_FWD_OUT(G, X, false)
    if (z) {
        if (xs) { SSMP_FWD_OUT_S(true, true); } else { SSMP_FWD_OUT_S(true, false); }
    } else {
        if (xs) { SSMP_FWD_OUT_S(false, true); } else { SSMP_FWD_OUT_S(false, false); }
    }
#undef SSMP_FWD_OUT_S
#undef SSMP_FWD_OUT
    SSMP_LAUNCH_CHECK();
    if (opt.hT) {
        const int64_t ND = (int64_t)NS * D;
        const int64_t n = (int64_t)opt.nseq * ND;
        k_empty_seq_states<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(opt.cu, opt.nseq, ND, opt.h0, opt.hT);
        SSMP_LAUNCH_CHECK();
    }
    return SSMP_OK;
}

template <typename T, int NS>
static int scan_dense_launch(const void* u, const void* delta, const float* A, const int32_t* pos,
                             const float* saved, int ci, float* ws, int64_t T_, int D, const ScanOpts& opt,
                             hipStream_t s) {
    const ScanWs L = scan_ws_layout(T_, D, NS, ci);
    const size_t ND = (size_t)NS * D;
    const float* start;
    size_t sstride;
    int G;
    if (ci == 0) {
        int st = scan_fwd_chunk_states<T, NS>(u, delta, A, pos, ws, L, T_, D, opt, s);
        if (st) return st;
        start = ws + L.hin;
        sstride = ND;
        G = fwd_chunk_len(T_, D);
    } else {
        // segments of at least 64 tokens, each from the kept state at its start
        G = ci > kLCMin ? ci : kLCMin;
        start = saved;
        sstride = (size_t)(G / ci) * ND;
    }
    const int64_t nseg = (T_ + G - 1) / G;
    const dim3 grid((unsigned)(L.ngroup * nseg));
    const int vec = stage_vec_ok<T>(D, {u, delta}) ? 1 : 0;
    const bool xs = opt.delta_bias != nullptr || opt.softplus != 0;
    const bool sv = opt.h0 != nullptr;
#define SSMP_REPLAY(X, S)                                                                                      \
    k_scan_fwd_replay<T, NS, X, S><<<grid, kWave, 0, s>>>((const T*)u, (const T*)delta, A, ws + L.bc, pos, start, \
                                                          sstride, ws + L.dense, T_, D, vec, G, opt)
    if (xs) {
        if (sv) SSMP_REPLAY(true, true); else SSMP_REPLAY(true, false);
    } else {
        if (sv) SSMP_REPLAY(false, true); else SSMP_REPLAY(false, false);
    }
#undef SSMP_REPLAY
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

template <typename T>
static int scan_fwd_dispatch(int N, const void* u, const void* delta, const float* A, const void* B, const void* C,
                             const float* Dskip, const void* z, const int32_t* pos, void* out, float* saved, int ci,
                             float* ws, int64_t T_, int D, const ScanOpts& o, hipStream_t s) {
#define SSMP_FWD_CASE(NV) \
    case NV: return scan_fwd_launch<T, NV>(u, delta, A, B, C, Dskip, z, pos, out, saved, ci, ws, T_, D, o, s);
    switch (N) {
        SSMP_FWD_CASE(1)
        SSMP_FWD_CASE(2)
        SSMP_FWD_CASE(4)
        SSMP_FWD_CASE(8)
        SSMP_FWD_CASE(16)
        default: return SSMP_ERR_UNSUPPORTED;
    }
#undef SSMP_FWD_CASE
}

int scan_dense_ckpt(int N, bool bf16, const void* u, const void* delta, const float* A, const int32_t* pos,
                    const float* saved, int ci, float* scratch, int64_t T, int D, const ScanOpts& o, hipStream_t s) {
#define SSMP_DENSE_CASE(NV)                                                                                     \
    case NV:                                                                                                    \
        return bf16 ? scan_dense_launch<uint16_t, NV>(u, delta, A, pos, saved, ci, scratch, T, D, o, s)         \
                    : scan_dense_launch<float, NV>(u, delta, A, pos, saved, ci, scratch, T, D, o, s);
    switch (N) {
        SSMP_DENSE_CASE(1)
        SSMP_DENSE_CASE(2)
        SSMP_DENSE_CASE(4)
        SSMP_DENSE_CASE(8)
        SSMP_DENSE_CASE(16)
        default: return SSMP_ERR_UNSUPPORTED;
    }
#undef SSMP_DENSE_CASE
}

}  // namespace ssmp

extern "C" size_t selective_scan_pack_saved_bytes(int64_t T, int32_t D, int32_t N, int32_t ckpt_interval) {
    if (T <= 0 || D <= 0 || N <= 0 || !ssmp::ck_interval_ok(ckpt_interval)) return 0;
    return ssmp::saved_floats(T, D, N, ckpt_interval) * sizeof(float);
}

extern "C" size_t selective_scan_pack_fwd_scratch_bytes(int64_t T, int32_t D, int32_t N) {
    if (T <= 0 || D <= 0 || N <= 0) return 0;
    return ssmp::scan_ws_layout(T, D, N, 0).fwd_total * sizeof(float);
}

extern "C" size_t selective_scan_pack_bwd_scratch_bytes(int64_t T, int32_t D, int32_t N, int32_t ckpt_interval) {
    if (T <= 0 || D <= 0 || N <= 0 || !ssmp::ck_interval_ok(ckpt_interval)) return 0;
    return ssmp::scan_ws_layout(T, D, N, ckpt_interval).bwd_total * sizeof(float);
}

extern "C" size_t selective_scan_pack_workspace_bytes(int64_t T, int32_t D, int32_t N) {
    if (T <= 0 || D <= 0 || N <= 0) return 0;
    const size_t f = selective_scan_pack_fwd_scratch_bytes(T, D, N);
    const size_t b = selective_scan_pack_bwd_scratch_bytes(T, D, N, ssmp::kCK);
    return selective_scan_pack_saved_bytes(T, D, N, ssmp::kCK) + (f > b ? f : b);
}

extern "C" int selective_scan_pack_fwd_ck(const void* u, const void* delta, const float* A, const void* B,
                                          const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                          void* out, int64_t T, int32_t D, int32_t N, int32_t dtype,
                                          const float* delta_bias, int32_t delta_softplus, float gate_floor,
                                          const int32_t* cu_seqlens, int32_t nseq, const float* initial_state,
                                          float* final_state, int32_t ckpt_interval, void* saved,
                                          size_t saved_bytes, void* scratch, size_t scratch_bytes, void* stream) {
    using namespace ssmp;
    int st = scan_check_args(T, D, N, dtype);
    if (st) return st;
    if (!ck_interval_ok(ckpt_interval)) return SSMP_ERR_SHAPE;
    const bool states = initial_state || final_state;
    if (states) {
        if (!cu_seqlens) return SSMP_ERR_NULL;
        if (nseq < 1 || (int64_t)nseq * D * N >= (int64_t(1) << 40)) return SSMP_ERR_SHAPE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    ScanOpts o{delta_bias, delta_softplus != 0 ? 1 : 0, gate_floor};
    if (states) {
        o.cu = cu_seqlens;
        o.nseq = nseq;
        o.h0 = initial_state;
        o.hT = final_state;
    }
    if (T == 0) {
        // every sequence is empty: it hands on its initial state
        if (!final_state) return SSMP_OK;
        const int64_t ND = (int64_t)D * N, n = (int64_t)nseq * ND;
        k_empty_seq_states<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(cu_seqlens, nseq, ND, initial_state,
                                                                       final_state);
        return hipGetLastError() == hipSuccess ? SSMP_OK : SSMP_ERR_HIP;
    }
    if (!u || !delta || !A || !B || !C || !pos || !out) return SSMP_ERR_NULL;
    if (ckpt_interval && (!saved || saved_bytes < selective_scan_pack_saved_bytes(T, D, N, ckpt_interval)))
        return SSMP_ERR_WORKSPACE;
    if (!scratch || scratch_bytes < selective_scan_pack_fwd_scratch_bytes(T, D, N)) return SSMP_ERR_WORKSPACE;
    float* sv = ckpt_interval ? static_cast<float*>(saved) : nullptr;
    float* ws = static_cast<float*>(scratch);
    return dtype == SSMP_BF16
               ? scan_fwd_dispatch<uint16_t>(N, u, delta, A, B, C, Dskip, z, pos, out, sv, ckpt_interval, ws, T, D,
                                             o, s)
               : scan_fwd_dispatch<float>(N, u, delta, A, B, C, Dskip, z, pos, out, sv, ckpt_interval, ws, T, D, o,
                                          s);
}

// ---------------------------------------------------------------------------
// The forward-only scan without allocation: its scratch lives in a buffer of
// the library's own, one per device, held until the process ends.
// ---------------------------------------------------------------------------
namespace ssmp {
constexpr size_t kNoAllocBytes = SSMP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kNoAllocBytes / sizeof(float)];

// The device address of `scratch` on each device, looked up once per device
// with that device current (host code must not use the array's name: it is
// a host-side stand-in, not a device address).
constexpr int kMaxDevices = 64;
static float* g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

static int noalloc_scratch(float** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSMP_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSMP_ERR_HIP;
        g_scratch[dev] = static_cast<float*>(p);
    }
    *out = g_scratch[dev];
    return SSMP_OK;
}
}  // namespace ssmp

extern "C" int selective_scan_pack_fwd_noalloc(const void* u, const void* delta, const float* A, const void* B,
                                               const void* C, const float* Dskip, const void* z,
                                               const int32_t* pos, void* out, int64_t T, int32_t D, int32_t N,
                                               int32_t dtype, const float* delta_bias, int32_t delta_softplus,
                                               float gate_floor, const int32_t* cu_seqlens, int32_t nseq,
                                               const float* initial_state, float* final_state, void* stream) {
    using namespace ssmp;
    int st = scan_check_args(T, D, N, dtype);
    if (st) return st;
    const size_t need = selective_scan_pack_fwd_scratch_bytes(T, D, N);
    if (need > kNoAllocBytes) return SSMP_ERR_TOO_LARGE;
    float* scr = nullptr;
    if (T > 0 && (st = noalloc_scratch(&scr))) return st;
    return selective_scan_pack_fwd_ck(u, delta, A, B, C, Dskip, z, pos, out, T, D, N, dtype, delta_bias,
                                      delta_softplus, gate_floor, cu_seqlens, nseq, initial_state, final_state, 0,
                                      nullptr, 0, scr, kNoAllocBytes, stream);
}

extern "C" int selective_scan_pack_fwd_states(const void* u, const void* delta, const float* A, const void* B,
                                              const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                              void* out, void* workspace, size_t workspace_bytes, int64_t T,
                                              int32_t D, int32_t N, int32_t dtype, const float* delta_bias,
                                              int32_t delta_softplus, float gate_floor, const int32_t* cu_seqlens,
                                              int32_t nseq, const float* initial_state, float* final_state,
                                              void* stream) {
    // the workspace: checkpoints every kCK tokens, then the scratch (a short
    // one is passed on as none, so that the argument checks come first)
    const size_t sb = selective_scan_pack_saved_bytes(T, D, N, ssmp::kCK);
    const bool ok = workspace && workspace_bytes >= selective_scan_pack_workspace_bytes(T, D, N);
    char* w = ok ? static_cast<char*>(workspace) : nullptr;
    return selective_scan_pack_fwd_ck(u, delta, A, B, C, Dskip, z, pos, out, T, D, N, dtype, delta_bias,
                                      delta_softplus, gate_floor, cu_seqlens, nseq, initial_state, final_state,
                                      ssmp::kCK, w, ok ? sb : 0, w ? w + sb : nullptr, ok ? workspace_bytes - sb : 0,
                                      stream);
}

extern "C" int selective_scan_pack_fwd_ex(const void* u, const void* delta, const float* A, const void* B,
                                          const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                          void* out, void* workspace, size_t workspace_bytes, int64_t T, int32_t D,
                                          int32_t N, int32_t dtype, const float* delta_bias, int32_t delta_softplus,
                                          float gate_floor, void* stream) {
    return selective_scan_pack_fwd_states(u, delta, A, B, C, Dskip, z, pos, out, workspace, workspace_bytes, T, D, N,
                                          dtype, delta_bias, delta_softplus, gate_floor, nullptr, 0, nullptr,
                                          nullptr, stream);
}

extern "C" int selective_scan_pack_fwd(const void* u, const void* delta, const float* A, const void* B,
                                       const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                       void* out, void* workspace, size_t workspace_bytes, int64_t T, int32_t D,
                                       int32_t N, int32_t dtype, void* stream) {
    return selective_scan_pack_fwd_ex(u, delta, A, B, C, Dskip, z, pos, out, workspace, workspace_bytes, T, D, N,
                                      dtype, nullptr, 0, 0.0f, stream);
}
