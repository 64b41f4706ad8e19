// selective_scan_pack backward.
//
// Shanghai AI Lab article on packed variable-length Mamba-1 training
// (gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), sections "SSM_pack算子" and
// "基本原理": the backward scan runs in reverse and, like the forward, no
// gradient crosses a head. With g = dout SiLU(z) and a_t = exp(delta_t A),
// per channel d and state n, t descending:
//   dh_t   = g_t C_t[n] + c_{t+1}            c_t = [t not a head] a_t dh_t
//   dC_t  += g_t h_t          dB_t += dh_t delta_t u_t      (summed over channels)
//   du_t   = g_t Dskip + delta_t sum_n dh_t B_t[n]
//   ddelta_t = u_t sum_n dh_t B_t[n] + sum_n [not head] A r_t,  r_t = dh_t a_t h_{t-1}
//   dA    += [not head] delta_t r_t                      dDskip += g_t u_t
//   dz_t   = dout_t y_t s (1 + z_t (1 - s)),  s = sigmoid(z_t)
// r_t is formed as c_t h_{t-1}: the carry a_t dh_t the step computes anyway,
// times the previous token's replayed state (the sub-chunk's entering state
// for its first token). With carried sequence states, h_{-1} of a head is its
// sequence's initial state and c_t there is that state's gradient.
//
// Time parallelism mirrors the forward, in reverse: a chunk's carry out of
// its first token is c_out = P' c_in + S' with
//   S' = sum_{s < first head} (prod_{r=t0..s} a_r) g_s C_s,  P' = prod a (0 if a head)
// which one forward sweep over the chunk's leading tokens yields. A
// sequential pass over chunks (right to left) turns these into the carry
// entering each chunk. The main kernel then walks each chunk backwards in
// kSub-token blocks: each block restarts from the forward's checkpoint at its
// first token and replays its tokens with their states and decays held in
// VGPRs before running the reverse step over them. A workgroup holds kCl * 64
// channels (kCl per lane) and splits the states between its waves (layout
// below); the sums over states are added across waves through LDS, and dB and
// dC (sums over channels) are added over the lane's channels in registers and
// over the wave's lanes through LDS, then written per channel group; dA and
// dDskip are written per chunk; small kernels finish all sums in a fixed
// order, so results are deterministic.
#include "scan_common.h"

#include <type_traits>

namespace ssmp {

// ---------------------------------------------------------------------------
// 1. reverse-carry summaries
// ---------------------------------------------------------------------------
// One block of the reverse-carry summary: for tokens s from the chunk start,
// sr += exp2(A2 * sum_{r<=s} delta_r) * g_s * C_s. The decay product is formed
// from a compensated running sum of delta (exact in real arithmetic).
// SAFE blocks stop at `nt`; fast blocks are full.
template <bool SAFE, bool GATE, typename T, int NS, int BT, typename St>
__device__ __forceinline__ void bsum_block(const T* lds, const float* __restrict__ bc, int64_t tb, int nt,
                                           const float (&A2)[NS], float (&sr)[NS], float& sdt, float& cdt,
                                           int lane, const StepMap& sm, float gf) {
    // the block's per-lane inputs are read from LDS before the first scalar
    // load: a wait for LDS data also waits for scalar loads in flight
    float dtv[BT], gv[BT];
#pragma unroll
    for (int k = 0; k < BT; ++k) {
        dtv[k] = St::get(lds, 0, k, lane);
        gv[k] = St::get(lds, 2, k, lane);
        if constexpr (GATE) {
            const float zz = St::get(lds, 1, k, lane);
            gv[k] *= __builtin_fmaf(zz, sigmoid_fast(zz), gf);
        }
    }
    if (sm.on) {
#pragma unroll
        for (int k = 0; k < BT; ++k) dtv[k] = sm.eff(dtv[k]);
    }
    const float* __restrict__ rows = bc + (size_t)tb * 2 * NS + NS;  // C rows
    float cur[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) cur[n] = rows[n];
#pragma unroll
    for (int k = 0; k < BT; ++k) {
        if constexpr (SAFE) {
            if (k >= nt) break;
        }
        float nxt[NS];
        const bool more = SAFE ? (k + 1 < nt) : (k + 1 < BT);
        scalar_loads_done();
        if (more) {
#pragma unroll
            for (int n = 0; n < NS; ++n) nxt[n] = rows[(k + 1) * 2 * NS + n];
        }
        __builtin_amdgcn_sched_barrier(0);  // the loads stay ahead of this token's arithmetic
        const float dt = dtv[k];
        const float g = gv[k];
        const float yk = dt - cdt;
        const float tk = sdt + yk;
        cdt = (tk - sdt) - yk;
        sdt = tk;
#pragma unroll
        for (int n = 0; n < NS; ++n) sr[n] = __builtin_fmaf(exp2_fast(A2[n] * sdt), g * cur[n], sr[n]);
        if (more) {
#pragma unroll
            for (int n = 0; n < NS; ++n) cur[n] = nxt[n];
        }
    }
}

template <typename T, int NS, bool GATE>
__global__ __launch_bounds__(64, 4) void k_scan_bwd_summary(const T* __restrict__ delta, const float* __restrict__ A,
                                                         const float* __restrict__ bc, const T* __restrict__ z,
                                                         const T* __restrict__ dout, const int32_t* __restrict__ pos,
                                                         float* __restrict__ Pr, float* __restrict__ Sr, int64_t T_,
                                                         int D, int vec, int lc, int logR, ScanOpts opt) {
    constexpr int BT = 8;
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
    // Only carries that reach the start of the main chunk (lc << logR tokens)
    // holding this sub-chunk are used: the sub-chunk's sequence must have
    // started before that point. Every other sub-chunk (one in the first main
    // chunk, at a head, or in a sequence starting inside its main chunk) is
    // skipped, and the carry pass counts it as a zero.
    if (!bwd_sum_needed(pos[t0], t0, logR, lc)) return;

    // first head in (t0, t1): the summary covers [t0, fh)
    int64_t fh = t1;
    for (int64_t base = t0; base < t1; base += kWave) {
        const int64_t t = base + lane;
        const bool f = (t < t1) && (t > t0) && pos[t] == 0;
        const uint64_t m = __ballot(f);
        if (m) {
            fh = base + __builtin_ctzll(m);
            break;
        }
    }
    float A2[NS], sr[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        A2[n] = A[(size_t)dd * NS + n] * kLog2e;
        sr[n] = 0.0f;
    }
    float sdt = 0.0f, cdt = 0.0f;
    const StepMap sm = step_map(opt, dd);
    const T* const src[3] = {delta, GATE ? z : delta, dout};
    St st;
    st.fetch(src, t0, T_, D, tl.g, lane, vec);
    for (int64_t tb = t0; tb < fh; tb += BT) {
        wave_sync();
        st.commit(lds, src, tb, T_, D, tl.g, lane, vec);
        wave_sync();
        if (tb + BT < fh) st.fetch(src, tb + BT, T_, D, tl.g, lane, vec);
        const int nt = (int)((tb + BT < fh) ? BT : fh - tb);
        if (nt == BT)
            bsum_block<false, GATE, T, NS, BT, St>(lds, bc, tb, BT, A2, sr, sdt, cdt, lane, sm, opt.gate_floor);
        else
            bsum_block<true, GATE, T, NS, BT, St>(lds, bc, tb, nt, A2, sr, sdt, cdt, lane, sm, opt.gate_floor);
    }
    if (opt.dhT && (fh < t1 || t1 == T_ || pos[t1] == 0)) {
        // the range ends at a sequence's last token: the carry entering that
        // token from the right is the sequence's final-state gradient, which
        // reaches the range's start through every decay of the range
        const float* __restrict__ gp = opt.dhT + ((size_t)seq_of(opt.cu, opt.nseq, fh - 1) * D + dd) * NS;
#pragma unroll
        for (int n = 0; n < NS; ++n) sr[n] = __builtin_fmaf(exp2_fast(A2[n] * sdt), gp[n], sr[n]);
    }
    if (act) {
        // the decay exp2(A2[n] * sdt) depends on n only through A: keep sdt
        // (NaN where a head cuts the sub-chunk, i.e. decay 0) per channel
        Pr[(size_t)c * D + d] = (fh < t1) ? __builtin_nanf("") : sdt;
#pragma unroll
        for (int n = 0; n < NS; ++n) Sr[((size_t)c * NS + n) * D + d] = sr[n];
    }
}

// ---------------------------------------------------------------------------
// 2. carries, right to left over the summary sub-chunks (lc tokens here; 2^logR
//    per main chunk): cin[m] = carry entering main chunk m from its right, i.e.
//    the carry entering its last sub-chunk
// ---------------------------------------------------------------------------
// Pr holds each sub-chunk's sum of delta per channel (NaN: a head cuts it).
template <int NS>
__global__ __launch_bounds__(256) void k_scan_bwd_carry(const float* __restrict__ Pr, const float* __restrict__ Sr,
                                                        const float* __restrict__ A,
                                                        const int32_t* __restrict__ pos, float* __restrict__ cin,
                                                        int D, int64_t nchunk, int lc, int logR) {
    const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ND = (int64_t)NS * D;
    const bool act = i0 < ND;
    const int64_t i = act ? i0 : ND - 1;  // lanes past the end run along (ballots need the wave) but store nothing
    // The summaries of kB chunks are loaded before the chain walks through
    // them, and the next kB are loaded while it does. Lane j < kB also loads
    // the position at the start of chunk cb - j (head test). Addresses step by
    // a fixed stride: the chain runs one wave per SIMD, so per-step index
    // arithmetic is not hidden by other waves.
    constexpr int kB = 16;
    const int lane = threadIdx.x % kWave;
    struct Batch {
        float P[kB], S[kB];
        int32_t used;  // lanes < kB: chunk cb - lane holds a summary
    };
    const int dch = (int)(i % D);
    const float A2 = A[(size_t)dch * NS + (int)(i / D)] * kLog2e;
    auto load = [&](Batch& b, int64_t cb) {
        const int64_t cj = cb - lane;
        b.used = (lane < kB && cj >= 0) ? (int32_t)bwd_sum_needed(pos[cj * lc], cj * lc, logR, lc) : 0;
        const float* p = Pr + (size_t)cb * D + dch;
        const float* q = Sr + (size_t)cb * ND + i;
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            if (cb - j >= 0) {
                b.P[j] = *p;
                b.S[j] = *q;
            } else {
                b.P[j] = 0.0f;
                b.S[j] = 0.0f;
            }
            p -= D;
            q -= ND;
        }
    };
    float cc = 0.0f;
    // main chunk c >> logR is entered from the right through its last
    // sub-chunk; the stores walk the main chunks from the last one down
    float* cp = cin + (size_t)((nchunk - 1) >> logR) * ND + i;
    const int64_t rmask = ((int64_t)1 << logR) - 1;
    Batch cur, nxt;
    load(cur, nchunk - 1);
    for (int64_t cb = nchunk - 1; cb >= 0; cb -= kB) {
        if (cb - kB >= 0) load(nxt, cb - kB);
        const uint64_t used = __ballot(cur.used != 0);  // bit j: chunk cb - j holds a summary
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const int64_t c = cb - j;
            if (c >= 0 && (((c + 1) & rmask) == 0 || c == nchunk - 1)) {
                if (act) *cp = cc;
                cp -= ND;
            }
            // skipped sub-chunks (heads among them) hand on zero; the select
            // keeps their unwritten summaries out, as in the forward
            const float tj = cur.P[j];
            const float Pj = (tj != tj) ? 0.0f : exp2_fast(A2 * tj);
            const float cn = !((used >> j) & 1u) ? 0.0f : (Pj == 0.0f) ? cur.S[j] : __builtin_fmaf(Pj, cc, cur.S[j]);
            cc = (c >= 0) ? cn : cc;
        }
        cur = nxt;
    }
}

// ---------------------------------------------------------------------------
// 3. the reverse pass
// ---------------------------------------------------------------------------
template <typename T>
struct BwdArgs {
    const T* u;
    const T* delta;
    const float* A;
    const float* bc;
    const float* Dskip;
    const T* z;
    const T* dout;
    const int32_t* pos;
    const float* ckpt;  // the state entering every 2^ckshift-th token (a multiple of kCK)
    int ckshift;
    const float* cin;
    T* du;
    T* ddelta;
    T* dz;
    float* dApart;
    float* dDpart;
    float* dbpart;
    float* dBC;
    float* sink;  // lanes with nothing to store write here, so that every path issues the same stores
    int64_t T_;
    int D;
    int lc;
    ScanOpts opt;
};

// Layout of the reverse pass. A workgroup covers kCl * 64 adjacent channels,
// kCl per lane (channels kCl*l .. kCl*l+kCl-1 of its group), and splits the
// states between its waves: wave q holds states q*NH .. q*NH+NH-1 of every
// channel, NH = min(N, 4), so SW = N / NH waves cover them all. A wave's
// registers then hold the states and decays of a whole block's replay,
// B_t[n] and C_t[n] are the same across the wave, and a lane's channels add
// their dB and dC terms in registers before the sums over channels go
// through LDS. One channel per lane over 8-token blocks measured faster (with
// the forward's checkpoint traffic halved) than two over 4-token blocks, at
// the same registers: the block's states and decays take K * kCl * NH each.
template <int NS>
struct Split {
    static constexpr int NH = NS < 4 ? NS : 4;
    static constexpr int SW = NS / NH;
};
constexpr int kCl = kBwdCl;                // channels per lane
constexpr int kGroupCh = kCl * kWave;      // channels per workgroup

// Tokens per block: the backward restarts from a state checkpoint at every
// block and replays it with its states in registers.
constexpr int kSub = kCK;

// Sum of v over groups of G consecutive lanes (G a power of two <= 16); every
// lane of a group receives the total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v += swap_adjacent(v);
    if constexpr (G >= 4)
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    if constexpr (G >= 8) v += __shfl_xor(v, 4);
    if constexpr (G >= 16) v += __shfl_xor(v, 8);
    return v;
}

// B_t and C_t of a block reach the arithmetic as DPP broadcasts: value j of
// a 16-value group sits in lane j of every 16-lane row of a VGPR, and
// row_newbcast:j hands it to all lanes as the first operand of the multiply or
// FMA that uses it, at no cost. Written as inline assembly because the
// compiler folds such broadcasts into multiplies only. A VALU write of a DPP
// source register needs two wait states before the DPP read; the broadcast
// registers are written by vector loads only, and a block's first read of
// each starts with s_nop 1 (NOP) in case a copy was placed just before it.
template <int J, bool NOP = false>
__device__ __forceinline__ void fmac_bc(float& acc, float src, float x) {
    if constexpr (NOP)
        asm("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
            : "+v"(acc) : "v"(src), "v"(x), "n"(J));
    else
        asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(acc) : "v"(src), "v"(x),
            "n"(J));
}
template <int J, bool NOP = false>
__device__ __forceinline__ float mul_bc(float src, float x) {
    float r;
    if constexpr (NOP)
        asm("s_nop 1\n\tv_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
            : "=v"(r) : "v"(src), "v"(x), "n"(J));
    else
        asm("v_mul_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "=v"(r) : "v"(src), "v"(x),
            "n"(J));
    return r;
}

// The block's B/C values of one wave: value v = kk*2NH + kind*NH + i (B for
// kind 0, C for kind 1, state q*NH + i, token tb + kk) in lane v % 16 of the
// rows of register v / 16.
template <int NS>
struct BcRegs {
    static constexpr int NH = Split<NS>::NH, K = kSub;
    static constexpr int V = K * 2 * NH;
    static constexpr int R = (V + 15) / 16;
    float r[R];
    // bc: fp32 rows [T][2N] (B then C); T < 2^31
    __device__ __forceinline__ void load(const float* __restrict__ bc, int tb, int T_, int q, int lane) {
        const int j = lane % 16;
        // the block's rows inside the tensor as a buffer resource: every lane
        // loads (no load waits behind a branch) at an offset that does not
        // change from block to block, and rows past the tensor read zeros
        // (tokens past the block's end are never used)
        const int nrow = (T_ - tb) < K ? (T_ - tb) : K;
        const auto rows = bytes_rsrc(bc + (size_t)tb * 2 * NS, (uint32_t)nrow * (uint32_t)(2 * NS * 4));
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const int v = k * 16 + j;
            const int kk = v / (2 * NH), kind = (v / NH) % 2, i = v % NH;
            const float x = Elt<float>::cvt(Elt<float>::raw_rsrc(rows, (uint32_t)((kk * 2 * NS + kind * NS + q * NH + i) * 4)));
            r[k] = (v < V) ? x : 0.0f;
        }
    }
};
template <int NS, int KK, int KIND, int I>
struct BcIdx {
    static constexpr int v = KK * 2 * Split<NS>::NH + KIND * Split<NS>::NH + I;
    static constexpr int reg = v / 16, lane = v % 16;
};

// Row stride (floats) of the per-lane dB/dC terms the sums over channels
// read: rows of 64 lanes, padded so that the float4 reads of two neighbouring
// rows by eight lanes fall on different banks.
constexpr int kXRow = kWave + 16;

// M floats that LDS moves in one access
template <int M>
struct alignas(4 * M) LdsVec {
    float v[M];
};
// What one block shares between the waves; blocks alternate between two of
// them, so that one barrier a block orders every access (see the block loop).
template <int NS>
struct BwdBuf {
    static constexpr int SW = Split<NS>::SW, K = kSub;
    LdsVec<2 * kCl> stp[K][kWave];    // per token, per lane: step and step*u of each of its channels
    LdsVec<kCl> gg[K][kWave];         // per token, per lane: g of each of its channels
    LdsVec<kCl> part[3][K][SW][kWave];  // per wave: y, sum_n dh B, sum_n A r of the lane's channels
};
template <int M>
__device__ __forceinline__ LdsVec<M> lds_vec(const float (&v)[M]) {
    LdsVec<M> r;
#pragma unroll
    for (int i = 0; i < M; ++i) r.v[i] = v[i];
    return r;
}

// LDS of a backward workgroup
template <int NS>
struct BwdShared {
    static constexpr int NH = Split<NS>::NH, SW = Split<NS>::SW;
    BwdBuf<NS> buf[2];
    // per wave, a token pair: dB and dC terms of its states (summed in
    // registers instead with 4 states a wave)
    float xb[NH == 4 ? 1 : SW][4 * NH][kXRow];
};

// Replay of a block from the state hin entering its first token: each
// token's states hh[kk] and decays ak[kk] (per channel of the lane), and this
// wave's share of y. SAFE blocks may be short (nb < K) or hold heads; fast
// blocks are neither.
// The block's per-token values of the lane's channels (step, step*u, g),
// read from LDS in one batch so that no token waits on its own read.
struct TokVals {
    float dt[kSub][kCl], dtu[kSub][kCl], gg[kSub][kCl];
};

template <bool SAFE, bool ST, int NS>
__device__ __forceinline__ void bwd_replay(BwdBuf<NS>& bf, const TokVals& tv, const BcRegs<NS>& bc, int nb,
                                           uint32_t heads, int lane, int q,
                                           const bool (&act)[kCl], const float (&A2)[kCl][Split<NS>::NH],
                                           const float (&hin)[kCl][Split<NS>::NH],
                                           float (&hh)[kSub][kCl][Split<NS>::NH],
                                           float (&ak)[kSub][kCl][Split<NS>::NH], const ScanOpts& opt, int64_t tb,
                                           int D, const int (&dd)[kCl]) {
    constexpr int NH = Split<NS>::NH, K = kSub;
    const int n0 = q * NH;
    float h[kCl][NH];
#pragma unroll
    for (int c = 0; c < kCl; ++c)
#pragma unroll
        for (int i = 0; i < NH; ++i) h[c][i] = hin[c][i];
    auto step = [&](auto KKc) {
        constexpr int kk = decltype(KKc)::value;
        const float(&dt)[kCl] = tv.dt[kk];
        const float(&dtu)[kCl] = tv.dtu[kk];
        if constexpr (SAFE) {
            if ((heads >> kk) & 1u) {
                asm volatile("");
#pragma unroll
                for (int c = 0; c < kCl; ++c) {
                    if (ST && opt.h0 && act[c]) {
                        const float* __restrict__ hp =
                            opt.h0 + ((size_t)seq_of(opt.cu, opt.nseq, tb + kk) * D + dd[c]) * NS + n0;
#pragma unroll
                        for (int i = 0; i < NH; ++i) h[c][i] = hp[i];
                    } else {
#pragma unroll
                        for (int i = 0; i < NH; ++i) h[c][i] = 0.0f;
                    }
                }
            }
        }
        float y[kCl];
        auto state = [&](auto Ic) {
            constexpr int i = decltype(Ic)::value;
            using Bi = BcIdx<NS, kk, 0, i>;
            using Ci = BcIdx<NS, kk, 1, i>;
            constexpr bool first = kk == 0 && i == 0;
#pragma unroll
            for (int c = 0; c < kCl; ++c) {
                const float a = exp2_fast(dt[c] * A2[c][i]);
                ak[kk][c][i] = a;
                const float b = (c == 0) ? mul_bc<Bi::lane, first>(bc.r[Bi::reg], dtu[c])
                                         : mul_bc<Bi::lane>(bc.r[Bi::reg], dtu[c]);
                h[c][i] = __builtin_fmaf(a, h[c][i], b);
                hh[kk][c][i] = h[c][i];
                if constexpr (i == 0) y[c] = mul_bc<Ci::lane>(bc.r[Ci::reg], h[c][i]);
                else fmac_bc<Ci::lane>(y[c], bc.r[Ci::reg], h[c][i]);
            }
        };
        static_for<NH>(state);
        bf.part[0][kk][q][lane] = lds_vec(y);
    };
    static_for_until<K>(step, SAFE ? nb : K);
}

// Sum over the 64 lanes of a wave of 16 values per lane, in registers. Each
// step folds two halves of the lanes onto each other and pairs two values,
// so the values per lane halve with the lanes each partial sum spans:
//  - 32-lane halves: v_permlane32_swap exchanges the upper half of one
//    register with the lower half of another, and the two results add up to
//    value j on lanes 0-31 and value j + 8 on lanes 32-63;
//  - 16-lane rows: v_permlane16_swap (odd rows of one register with even rows
//    of the other), likewise;
//  - 8- and 4-lane halves of a row: a DPP rotate by 8, or shift by 4, adds
//    each lane's partner, and the bank mask keeps the half that holds the
//    value;
//  - the four lanes of a quad: two DPP adds.
// Lane l ends with the total of value l / 4. The swaps are inline assembly
// (the compiler's builtins for them return the first register twice), and so
// are the DPP adds, for the bank masks. Each block first waits the two states
// a swap or DPP read needs after a VALU write of its source, and the last
// waits them after itself, since the compiler does not count inline assembly
// as VALU.
__device__ __forceinline__ float wave_sum16(const float (&v)[16]) {
    float w[16], x[4], y[2], z;
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = v[j];
    // after a swap of (a, b): a = (a lo, b lo), b = (a hi, b hi). One wait
    // state pair first: a swap reading a register a VALU just wrote needs them.
    asm("s_nop 1\n\t"
        "v_permlane32_swap_b32 %0, %8\n\tv_permlane32_swap_b32 %1, %9\n\t"
        "v_permlane32_swap_b32 %2, %10\n\tv_permlane32_swap_b32 %3, %11\n\t"
        "v_permlane32_swap_b32 %4, %12\n\tv_permlane32_swap_b32 %5, %13\n\t"
        "v_permlane32_swap_b32 %6, %14\n\tv_permlane32_swap_b32 %7, %15"
        : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]), "+v"(w[6]), "+v"(w[7]),
          "+v"(w[8]), "+v"(w[9]), "+v"(w[10]), "+v"(w[11]), "+v"(w[12]), "+v"(w[13]), "+v"(w[14]), "+v"(w[15]));
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] += w[j + 8];
    // odd rows of the first with even rows of the second
    asm("s_nop 1\n\t"
        "v_permlane16_swap_b32 %0, %4\n\tv_permlane16_swap_b32 %1, %5\n\t"
        "v_permlane16_swap_b32 %2, %6\n\tv_permlane16_swap_b32 %3, %7"
        : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]), "+v"(w[6]), "+v"(w[7]));
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = w[j] + w[j + 4];
    // x[j]: value j + 4 * (l / 16). y[j]: value j (lanes 0-7 of a row) or j + 2 (lanes 8-15) + 4 * row
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3" : "=v"(y[j]) : "v"(x[j]));
        asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0xc" : "+v"(y[j]) : "v"(x[j + 2]));
    }
    // z: value l / 4 (lanes 0-3 and 8-11 of a row take lane + 4, the others lane - 4)
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_shl:4 row_mask:0xf bank_mask:0x5" : "=v"(z) : "v"(y[0]));
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_shr:4 row_mask:0xf bank_mask:0xa\n\ts_nop 1" : "+v"(z) : "v"(y[1]));
    return group_sum<4>(z);
}

// Reverse step over the block, a token pair at a time; after each pair, dB
// (kind 0: sum over channels of dh * step*u) and dC (kind 1: of g * h) of its
// two tokens. A lane's channels are added in registers, then each value over
// the wave's lanes: with 4 states a wave (16 values a pair) by wave_sum16;
// with fewer, by LPO lanes reading the terms the wave left in LDS.
template <bool SAFE, bool ST, int NS>
__device__ __forceinline__ void bwd_reverse(BwdBuf<NS>& bf, float* __restrict__ myx, const TokVals& tv,
                                            const BcRegs<NS>& bc, int nb, uint32_t heads, int lane, int q,
                                            const bool (&act)[kCl], const float (&A2)[kCl][Split<NS>::NH],
                                            const float (&hin)[kCl][Split<NS>::NH],
                                            const float (&hh)[kSub][kCl][Split<NS>::NH],
                                            const float (&ak)[kSub][kCl][Split<NS>::NH],
                                            float (&carry)[kCl][Split<NS>::NH], float (&dA)[kCl][Split<NS>::NH],
                                            float* __restrict__ dbc_row, float* __restrict__ sink, const ScanOpts& opt, int64_t tb, int D,
                                            const int (&dd)[kCl]) {
    constexpr int NH = Split<NS>::NH, K = kSub;
    constexpr bool kRegSum = NH == 4;
    constexpr int LPO = kWave / (4 * NH);  // lanes adding up one dB/dC value of a token pair
    constexpr int CPL = kWave / LPO;       // lanes' terms each of them adds
    static_assert(K % 2 == 0 && CPL % 4 == 0, "tiling");
    const int n0 = q * NH;
    float xr[2][2][NH];  // a pair's dB/dC terms: [token][kind][state]
    auto put = [&](int tk, int kind, int i, float v) {
        if constexpr (kRegSum) xr[tk][kind][i] = v;
        else myx[((tk * 2 + kind) * NH + i) * kXRow + lane] = v;
    };
    auto tok = [&](auto KKc) {
        constexpr int kk = decltype(KKc)::value;
        constexpr int tk = kk % 2;
        if constexpr (SAFE) {
            if (kk >= nb) return;
        }
        const float(&dt)[kCl] = tv.dt[kk];
        const float(&dtu)[kCl] = tv.dtu[kk];
        const float(&gg)[kCl] = tv.gg[kk];
        float sumB[kCl], sumAr[kCl];
#pragma unroll
        for (int c = 0; c < kCl; ++c) sumAr[c] = 0.0f;
        if (SAFE && ((heads >> kk) & 1u)) {
            asm volatile("");
            // With states, what the decay passes back out of the head is the
            // initial state's gradient, the initial state is the previous
            // state of the r term, and the carry into the token before the
            // head (the previous sequence's last) is that sequence's
            // final-state gradient.
            const bool st = ST && (opt.h0 || opt.dh0);
            const int64_t t = tb + kk;
            const int s_here = st ? seq_of(opt.cu, opt.nseq, t) : 0;
            const int s_prev = (ST && opt.dhT && t > 0) ? seq_of(opt.cu, opt.nseq, t - 1) : 0;
            auto state = [&](auto Ic) {
                constexpr int i = decltype(Ic)::value;
                using Bi = BcIdx<NS, kk, 0, i>;
                using Ci = BcIdx<NS, kk, 1, i>;
                float xB = 0.0f, xC = 0.0f;
#pragma unroll
                for (int c = 0; c < kCl; ++c) {
                    fmac_bc<Ci::lane>(carry[c][i], bc.r[Ci::reg], gg[c]);
                    const float dh = carry[c][i];
                    if constexpr (i == 0) sumB[c] = mul_bc<Bi::lane>(bc.r[Bi::reg], dh);
                    else fmac_bc<Bi::lane>(sumB[c], bc.r[Bi::reg], dh);
                    xB = __builtin_fmaf(dh, dtu[c], xB);
                    xC = __builtin_fmaf(gg[c], hh[kk][c][i], xC);
                    if (st) {
                        const size_t so = ((size_t)s_here * D + dd[c]) * NS + n0 + i;
                        const float cr = ak[kk][c][i] * dh;
                        if (opt.h0) {
                            const float r = cr * (act[c] ? opt.h0[so] : 0.0f);
                            sumAr[c] = __builtin_fmaf(r, A2[c][i], sumAr[c]);
                            dA[c][i] = __builtin_fmaf(r, dt[c], dA[c][i]);
                        }
                        if (opt.dh0 && act[c]) opt.dh0[so] = cr;
                    }
                    const bool gp = ST && opt.dhT && t > 0 && act[c];
                    carry[c][i] = gp ? opt.dhT[((size_t)s_prev * D + dd[c]) * NS + n0 + i] : 0.0f;
                }
                put(tk, 0, i, xB);
                put(tk, 1, i, xC);
            };
            static_for<NH>(state);
        } else {
            auto state = [&](auto Ic) {
                constexpr int i = decltype(Ic)::value;
                using Bi = BcIdx<NS, kk, 0, i>;
                using Ci = BcIdx<NS, kk, 1, i>;
                constexpr bool first = kk == K - 1 && i == 0;
                float xB = 0.0f, xC = 0.0f;
#pragma unroll
                for (int c = 0; c < kCl; ++c) {
                    // dh = carry + g C, formed in the carry's own register
                    if (c == 0) fmac_bc<Ci::lane, first>(carry[c][i], bc.r[Ci::reg], gg[c]);
                    else fmac_bc<Ci::lane>(carry[c][i], bc.r[Ci::reg], gg[c]);
                    const float dh = carry[c][i];
                    if constexpr (i == 0) sumB[c] = mul_bc<Bi::lane>(bc.r[Bi::reg], dh);
                    else fmac_bc<Bi::lane>(sumB[c], bc.r[Bi::reg], dh);
                    xB = __builtin_fmaf(dh, dtu[c], xB);
                    xC = __builtin_fmaf(gg[c], hh[kk][c][i], xC);
                    // carry to t-1: a_t dh_t; r = dh_t a_t h_{t-1}
                    carry[c][i] = ak[kk][c][i] * dh;
                    const float r = carry[c][i] * (kk == 0 ? hin[c][i] : hh[kk > 0 ? kk - 1 : 0][c][i]);
                    sumAr[c] = __builtin_fmaf(r, A2[c][i], sumAr[c]);
                    dA[c][i] = __builtin_fmaf(r, dt[c], dA[c][i]);
                }
                put(tk, 0, i, xB);
                put(tk, 1, i, xC);
            };
            static_for<NH>(state);
        }
        bf.part[1][kk][q][lane] = lds_vec(sumB);
        bf.part[2][kk][q][lane] = lds_vec(sumAr);
    };
    // where lane's total of a pair goes: value o = lane / LPO, i.e. token tk,
    // kind, state oi of the pair
    const int o = lane / LPO;
    const int tk = o / (2 * NH), kind = (o / NH) % 2, oi = o % NH;
    auto store = [&](int kp, float acc) {
        const int kk = 2 * kp + tk;
        // every lane of the output stores the same value: no lane-dependent branch
        float* dst = (!SAFE || kk < nb) ? dbc_row + (size_t)kk * 2 * NS + kind * NS + n0 + oi : sink + lane;
        *dst = acc;
    };
    if constexpr (kRegSum) {
        auto pair = [&](auto KPc) {
            constexpr int kp = K / 2 - 1 - decltype(KPc)::value;  // pairs right to left
            if constexpr (SAFE) {
                // tokens past a short block leave their terms unset; their
                // totals go to the sink
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                        for (int i = 0; i < NH; ++i) xr[t2][k2][i] = 0.0f;
            }
            tok(std::integral_constant<int, 2 * kp + 1>{});
            tok(std::integral_constant<int, 2 * kp>{});
            float v[16];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                    for (int i = 0; i < NH; ++i) v[(t2 * 2 + k2) * NH + i] = xr[t2][k2][i];
            store(kp, wave_sum16(v));
        };
        static_for<K / 2>(pair);
    } else {
        // The terms of a pair are read back right after they are written and
        // added up after the next pair's reverse step: a wave's LDS accesses
        // complete in issue order, so the next pair's writes cannot overtake
        // the reads, and the reads' latency hides behind that step. The LPO
        // lanes of an output read interleaved float4s: together a contiguous
        // run, conflict-free.
        const float4* __restrict__ xv =
            reinterpret_cast<const float4*>(myx + ((tk * 2 + kind) * NH + oi) * kXRow) + lane % LPO;
        float4 rx[CPL / 4];
        auto finish = [&](int kp) {
            float acc;
#pragma unroll
            for (int m = 0; m < CPL / 4; ++m) {
                const float s4 = (rx[m].x + rx[m].y) + (rx[m].z + rx[m].w);
                acc = (m == 0) ? s4 : acc + s4;
            }
            store(kp, group_sum<LPO>(acc));
        };
        auto pair = [&](auto KPc) {
            constexpr int kp = K / 2 - 1 - decltype(KPc)::value;  // pairs right to left
            tok(std::integral_constant<int, 2 * kp + 1>{});
            tok(std::integral_constant<int, 2 * kp>{});
            if constexpr (kp + 1 < K / 2) finish(kp + 1);
            wave_sync();
#pragma unroll
            for (int m = 0; m < CPL / 4; ++m) rx[m] = xv[m * LPO];
            wave_sync();
        };
        static_for<K / 2>(pair);
        finish(0);
    }
}

// The reverse pass over one chunk. Per kSub-token block, right to left:
//  1. prologue: each wave maps the step, gate and their products for every
//     SW-th token of the block (its own tokens) and shares them through LDS;
//  2. replay: every wave runs its states through the block from the
//     checkpoint at the block start, keeping each token's state and decay;
//  3. reverse step with the block's dB and dC (bwd_reverse), written as this
//     channel group's partial rows;
//  4. epilogue: each wave finishes its own tokens: the per-wave sums over
//     states (y, sum dh B, sum A r) are added in wave order, and du, ddelta
//     and dz are stored.
// Heads reset the replayed state and cut the reverse carry; with carried
// states, a head starts from its sequence's h0 (replay), passes a * dh out as
// dh0 and restarts the carry from the previous sequence's dhT (reverse).
template <typename T, int NS, bool GATE, bool XS, bool ST>
__global__ __launch_bounds__(kWave * Split<NS>::SW, 2) void k_scan_bwd_main(
    BwdArgs<T> p, const float* __restrict__ bcp) {
    constexpr int NH = Split<NS>::NH, SW = Split<NS>::SW, K = kSub, KQ = K / SW;
    static_assert(K % SW == 0, "tiling");
    __shared__ __attribute__((aligned(16))) BwdShared<NS> sh;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int q = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int D = p.D;
    const int64_t T_ = p.T_;
    const unsigned ngroup = (unsigned)((D + kGroupCh - 1) / kGroupCh);
    const int g = (int)(blockIdx.x % ngroup);
    const int64_t c_ = blockIdx.x / ngroup;
    int d[kCl], dd[kCl];
    bool act[kCl];
#pragma unroll
    for (int c = 0; c < kCl; ++c) {
        d[c] = g * kGroupCh + kCl * lane + c;
        act[c] = d[c] < D;
        dd[c] = act[c] ? d[c] : D - 1;
    }
    uint32_t bo[kCl];  // byte offsets of the lane's channels in a (T, D) row
#pragma unroll
    for (int c = 0; c < kCl; ++c) bo[c] = (uint32_t)dd[c] * (uint32_t)sizeof(T);
    const int64_t t0 = c_ * p.lc;
    const int64_t t1 = (t0 + p.lc < T_) ? t0 + p.lc : T_;
    const size_t ND = (size_t)NS * D;
    const int n0 = q * NH;

    float A2[kCl][NH], carry[kCl][NH], dA[kCl][NH];
#pragma unroll
    for (int c = 0; c < kCl; ++c)
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            A2[c][i] = p.A[(size_t)dd[c] * NS + n0 + i] * kLog2e;
            carry[c][i] = act[c] ? p.cin[(size_t)c_ * ND + (size_t)(n0 + i) * D + dd[c]] : 0.0f;
            dA[c][i] = 0.0f;
        }
    if (ST && p.opt.dhT && (t1 == T_ || p.pos[t1] == 0)) {
        // the chunk ends at a sequence's last token (the carry pass hands it
        // zero): it starts from that sequence's final-state gradient
        const int s = seq_of(p.opt.cu, p.opt.nseq, t1 - 1);
#pragma unroll
        for (int c = 0; c < kCl; ++c)
            if (act[c]) {
#pragma unroll
                for (int i = 0; i < NH; ++i) carry[c][i] = p.opt.dhT[((size_t)s * D + dd[c]) * NS + n0 + i];
            }
    }
    float Dv[kCl], dDacc[kCl], dbacc[kCl];
#pragma unroll
    for (int c = 0; c < kCl; ++c) dDacc[c] = dbacc[c] = 0.0f;
    StepMap sm[kCl];
#pragma unroll
    for (int c = 0; c < kCl; ++c) {
        Dv[c] = (p.Dskip && act[c]) ? p.Dskip[dd[c]] : 0.0f;
        sm[c] = step_map(p.opt, dd[c]);
    }
    const float gf = p.opt.gate_floor;

    // Inputs of a block, loaded two blocks ahead into one of two buffers
    // (the block loop is unrolled by two, so neither is ever copied): this
    // wave's own tokens (every SW-th, from q), raw, for both channels; the
    // checkpoint at the block start; the block's B/C values.
    struct Pre {
        uint32_t ru[KQ][kCl], rd[KQ][kCl], rz[KQ][kCl], rg[KQ][kCl];  // raw bits
        float hn[kCl][NH];
        BcRegs<NS> bc;
        int32_t pos;  // lanes < K: position of token tb + lane (0 past the tensor)
    };
    Pre pre[2];
    // token indices in 32 bits (T < 2^31): their compares and selects stay
    // on the scalar unit
    const int T32 = (int)T_;
    auto prefetch = [&](Pre& b, int64_t tb) {
        // every load is issued on every path, so the waits for them can count
        // the operations after them: a row past the tensor is an empty buffer
        // resource and reads zeros
        const int tb32 = (int)tb;
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
            const int t = tb32 + q + j * SW;
            const bool in = t < T32;
            const size_t rb = (size_t)(in ? t : 0) * (size_t)D;
            const uint32_t nbytes = in ? (uint32_t)D * (uint32_t)sizeof(T) : 0u;
            const auto ru = bytes_rsrc(p.u + rb, nbytes), rd = bytes_rsrc(p.delta + rb, nbytes);
            const auto rg = bytes_rsrc(p.dout + rb, nbytes);
            const auto rz = bytes_rsrc(GATE ? p.z + rb : p.u, GATE ? nbytes : 0u);
#pragma unroll
            for (int c = 0; c < kCl; ++c) {
                b.ru[j][c] = Elt<T>::raw_rsrc(ru, bo[c]);
                b.rd[j][c] = Elt<T>::raw_rsrc(rd, bo[c]);
                b.rz[j][c] = GATE ? Elt<T>::raw_rsrc(rz, bo[c]) : 0u;
                b.rg[j][c] = Elt<T>::raw_rsrc(rg, bo[c]);
            }
        }
        const float* __restrict__ slot = p.ckpt + ((uint64_t)tb >> p.ckshift) * ND;  // tb >= 0
#pragma unroll
        for (int c = 0; c < kCl; ++c) ck_load<NS, NH>(slot, dd[c], D, n0, true, b.hn[c]);
        b.bc.load(bcp, tb32, T32, q, lane);
        const int np = (T32 - tb32) < kWave ? (T32 - tb32) : kWave;
        b.pos = (int32_t)Elt<float>::raw_rsrc(bytes_rsrc(p.pos + tb, (uint32_t)np * 4u), (uint32_t)lane * 4u);
    };

    // The per-block work in three parts: the prologue maps this wave's own
    // tokens (every SW-th) and shares them through bf; the main part replays
    // the block and runs the reverse step, leaving the per-wave sums in bf and
    // refilling b with the inputs of block jb - 2; the epilogue adds those
    // sums for the wave's own tokens and stores their gradients.
    // The loop runs main(jb), prologue(jb - 1), one barrier, epilogue(jb), so
    // with blocks alternating between the two bf buffers one barrier a block
    // orders every shared access: prologue(jb - 1) writes the buffer that
    // main(jb + 1) read before the previous barrier, main(jb - 1) reads it
    // after this one, and the per-wave sums of main(jb) are read after this
    // barrier and written again (by main(jb - 2)) after the next one.
    struct EVals {
        float u[KQ][kCl], dt[KQ][kCl], gg[KQ][kCl], fz[KQ][kCl], sl[KQ][kCl];  // fz: dz = (y + Dskip u) fz
    };
    auto block_nb = [&](int64_t jb) {
        const int64_t tb = t0 + jb * K;
        return (int)(((tb + K < t1) ? tb + K : t1) - tb);
    };
    auto prologue = [&](const Pre& b, int64_t jb, BwdBuf<NS>& bf, EVals& ev) {
        const int nb = block_nb(jb);
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
            const int kk = q + j * SW;
            float dtv[kCl], dtu[kCl], ggv[kCl];
#pragma unroll
            for (int c = 0; c < kCl; ++c) {
                const bool v = act[c] && kk < nb;
                const float rdv = Elt<T>::cvt(b.rd[j][c]), rzv = Elt<T>::cvt(b.rz[j][c]);
                const float rgv = Elt<T>::cvt(b.rg[j][c]);
                float sl = 1.0f;
                float dt = XS ? sm[c].eff(rdv, sl) : rdv;
                dt = v ? dt : 0.0f;  // lanes past D and tokens past the block replay zeros
                const float uu = v ? Elt<T>::cvt(b.ru[j][c]) : 0.0f;
                float gg = rgv, fz = 0.0f;
                if constexpr (GATE) {
                    const float sg = sigmoid_fast(rzv);
                    gg *= __builtin_fmaf(rzv, sg, gf);
                    fz = rgv * sg * (1.0f + rzv * (1.0f - sg));
                }
                gg = v ? gg : 0.0f;
                dtv[c] = dt; dtu[c] = dt * uu; ggv[c] = gg;
                ev.u[j][c] = uu; ev.dt[j][c] = dt; ev.gg[j][c] = gg; ev.fz[j][c] = fz; ev.sl[j][c] = sl;
            }
            float sv[2 * kCl];
#pragma unroll
            for (int c = 0; c < kCl; ++c) {
                sv[2 * c] = dtv[c];
                sv[2 * c + 1] = dtu[c];
            }
            bf.stp[kk][lane] = lds_vec(sv);
            bf.gg[kk][lane] = lds_vec(ggv);
        }
    };
    auto main_part = [&](Pre& b, int64_t jb, BwdBuf<NS>& bf) {
        const int64_t tb = t0 + jb * K;
        const int nb = block_nb(jb);
        // head flags of the block, from the prefetched positions: bit k for token tb + k
        const int hl = (T32 - (int)tb) < K ? (T32 - (int)tb) : K;  // the block's tokens inside the tensor
        const uint32_t heads = (uint32_t)__ballot(lane < hl && b.pos == 0);
        float hh[K][kCl][NH], ak[K][kCl][NH];
        TokVals tv;
#pragma unroll
        for (int kk = 0; kk < K; ++kk) {
            const LdsVec<2 * kCl> st = bf.stp[kk][lane];
            const LdsVec<kCl> g2 = bf.gg[kk][lane];
#pragma unroll
            for (int c = 0; c < kCl; ++c) {
                tv.dt[kk][c] = st.v[2 * c];
                tv.dtu[kk][c] = st.v[2 * c + 1];
                tv.gg[kk][c] = g2.v[c];
            }
        }
        float* __restrict__ dbc_row = p.dBC + ((size_t)g * T_ + tb) * 2 * NS;
        float* __restrict__ myx = &sh.xb[NH == 4 ? 0 : q][0][0];
        if (heads == 0 && nb == K) {
            bwd_replay<false, ST, NS>(bf, tv, b.bc, nb, heads, lane, q, act, A2, b.hn, hh, ak, p.opt, tb, D, dd);
            bwd_reverse<false, ST, NS>(bf, myx, tv, b.bc, nb, heads, lane, q, act, A2, b.hn, hh, ak, carry, dA,
                                       dbc_row, p.sink, p.opt, tb, D, dd);
        } else {
            bwd_replay<true, ST, NS>(bf, tv, b.bc, nb, heads, lane, q, act, A2, b.hn, hh, ak, p.opt, tb, D, dd);
            bwd_reverse<true, ST, NS>(bf, myx, tv, b.bc, nb, heads, lane, q, act, A2, b.hn, hh, ak, carry, dA,
                                      dbc_row, p.sink, p.opt, tb, D, dd);
        }
        prefetch(b, tb >= t0 + 2 * K ? tb - 2 * K : t0);  // past the chunk start: a dummy reload
    };
    auto epilogue = [&](int64_t jb, const BwdBuf<NS>& bf, const EVals& ev) {
        const int64_t tb = t0 + jb * K;
        const int nb = block_nb(jb);
#pragma unroll
        for (int j = 0; j < KQ; ++j) {
            const int kk = q + j * SW;
            const bool tok = kk < nb;  // tokens past the block store nothing
            LdsVec<kCl> y = bf.part[0][kk][0][lane], sB = bf.part[1][kk][0][lane], sA = bf.part[2][kk][0][lane];
#pragma unroll
            for (int w = 1; w < SW; ++w) {
                const LdsVec<kCl> a = bf.part[0][kk][w][lane], bb = bf.part[1][kk][w][lane],
                                  cc = bf.part[2][kk][w][lane];
#pragma unroll
                for (int c = 0; c < kCl; ++c) {
                    y.v[c] += a.v[c];
                    sB.v[c] += bb.v[c];
                    sA.v[c] += cc.v[c];
                }
            }
            const float(&yv)[kCl] = y.v;
            const float(&sBv)[kCl] = sB.v;
            const float(&sAv)[kCl] = sA.v;
            // the token's rows as buffer resources: a token past the block gets
            // empty ones, a lane past D an offset past the row; both stores drop
            const size_t rb = (size_t)(tok ? tb + kk : 0) * D;
            const uint32_t rowb = tok ? (uint32_t)D * (uint32_t)sizeof(T) : 0u;
            const auto rdu = bytes_rsrc(p.du + rb, rowb), rdd = bytes_rsrc(p.ddelta + rb, rowb);
            const auto rdz = bytes_rsrc(GATE ? p.dz + rb : p.du, GATE ? rowb : 0u);
#pragma unroll
            for (int c = 0; c < kCl; ++c) {
                const float uu = ev.u[j][c];
                const float yy = __builtin_fmaf(Dv[c], uu, yv[c]);
                const float duv = __builtin_fmaf(ev.gg[j][c], Dv[c], ev.dt[j][c] * sBv[c]);
                float ddv = __builtin_fmaf(uu, sBv[c], sAv[c] * kLn2);
                if constexpr (XS) {
                    ddv *= ev.sl[j][c];  // with respect to the stored step
                    dbacc[c] += (tok && act[c]) ? ddv : 0.0f;
                }
                dDacc[c] = __builtin_fmaf(ev.gg[j][c], uu, dDacc[c]);
                const float dzv = yy * ev.fz[j][c];
                const uint32_t o = (uint32_t)d[c] * (uint32_t)sizeof(T);
                Elt<T>::st_rsrc(rdu, o, duv);
                Elt<T>::st_rsrc(rdd, o, ddv);
                if constexpr (GATE) Elt<T>::st_rsrc(rdz, o, dzv);
            }
        }
    };

    // blocks right to left; block jb uses pre[(nblk - 1 - jb) % 2], buf and
    // e-values of the same parity
    const int64_t nblk = (t1 - t0 + K - 1) / K;
    prefetch(pre[0], t0 + (nblk - 1) * K);
    prefetch(pre[1], nblk >= 2 ? t0 + (nblk - 2) * K : t0);
    if constexpr (SW == 1) {
        // one wave: its barriers cost nothing, and one set of e-values keeps
        // its registers
        EVals ev;
        for (int64_t jb = nblk - 1; jb >= 0; jb -= 2) {
            prologue(pre[0], jb, sh.buf[0], ev);
            __syncthreads();
            main_part(pre[0], jb, sh.buf[0]);
            __syncthreads();
            epilogue(jb, sh.buf[0], ev);
            if (jb == 0) break;
            __syncthreads();
            prologue(pre[1], jb - 1, sh.buf[0], ev);
            __syncthreads();
            main_part(pre[1], jb - 1, sh.buf[0]);
            __syncthreads();
            epilogue(jb - 1, sh.buf[0], ev);
            __syncthreads();
        }
    } else {
        EVals ev[2];
        prologue(pre[0], nblk - 1, sh.buf[0], ev[0]);
        __syncthreads();
        for (int64_t jb = nblk - 1; jb >= 0; jb -= 2) {
            main_part(pre[0], jb, sh.buf[0]);
            if (jb >= 1) prologue(pre[1], jb - 1, sh.buf[1], ev[1]);
            __syncthreads();
            epilogue(jb, sh.buf[0], ev[0]);
            if (jb == 0) break;
            main_part(pre[1], jb - 1, sh.buf[1]);
            if (jb >= 2) prologue(pre[0], jb - 2, sh.buf[0], ev[0]);
            __syncthreads();
            epilogue(jb - 1, sh.buf[1], ev[1]);
        }
    }

    // per-chunk partial sums: dA per state; dD and d bias added over the waves in order
#pragma unroll
    for (int c = 0; c < kCl; ++c)
        if (act[c]) {
#pragma unroll
            for (int i = 0; i < NH; ++i) p.dApart[(size_t)c_ * ND + (size_t)(n0 + i) * D + d[c]] = dA[c][i];
        }
    __syncthreads();
    sh.buf[0].part[0][0][q][lane] = lds_vec(dDacc);
    sh.buf[0].part[1][0][q][lane] = lds_vec(dbacc);
    __syncthreads();
    if (q == 0) {
        float sDv[kCl], sbv[kCl];
#pragma unroll
        for (int c = 0; c < kCl; ++c) sDv[c] = sbv[c] = 0.0f;
#pragma unroll
        for (int w = 0; w < SW; ++w) {
            const LdsVec<kCl> a = sh.buf[0].part[0][0][w][lane], b = sh.buf[0].part[1][0][w][lane];
#pragma unroll
            for (int c = 0; c < kCl; ++c) {
                sDv[c] += a.v[c];
                sbv[c] += b.v[c];
            }
        }
#pragma unroll
        for (int c = 0; c < kCl; ++c)
            if (act[c]) {
                p.dDpart[(size_t)c_ * D + d[c]] = sDv[c];
                if (XS) p.dbpart[(size_t)c_ * D + d[c]] = sbv[c];
            }
    }
}

// ---------------------------------------------------------------------------
// 4. fixed-order sums
// ---------------------------------------------------------------------------
template <int NS>
__global__ __launch_bounds__(256) void k_scan_bwd_reduce_params(const float* __restrict__ dApart,
                                                                const float* __restrict__ dDpart,
                                                                const float* __restrict__ dbpart, int64_t nchunk,
                                                                int D, float* __restrict__ dA,
                                                                float* __restrict__ dD, float* __restrict__ dbias) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // n*D + d
    const int64_t ND = (int64_t)NS * D;
    if (i < ND) {
        const float acc = ordered_sum(dApart + i, nchunk, (size_t)ND);
        const int n = (int)(i / D), d = (int)(i % D);
        dA[(size_t)d * NS + n] = acc;
    }
    if (dD && i < D) dD[i] = ordered_sum(dDpart + i, nchunk, (size_t)D);
    if (dbias && i < D) dbias[i] = ordered_sum(dbpart + i, nchunk, (size_t)D);
}

template <int NS>
__global__ __launch_bounds__(256) void k_scan_bwd_reduce_bc(const float* __restrict__ dBC, int64_t ngroup,
                                                            int64_t T_, float* __restrict__ dB,
                                                            float* __restrict__ dC) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // t*2NS + j
    if (i >= T_ * 2 * NS) return;
    const float acc = ordered_sum<8>(dBC + i, ngroup, (size_t)T_ * 2 * NS);
    const int64_t t = i / (2 * NS);
    const int j = (int)(i % (2 * NS));
    if (j < NS) dB[t * NS + j] = acc;
    else dC[t * NS + (j - NS)] = acc;
}

template <typename T, int NS>
static int scan_bwd_launch(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, const int32_t* pos, const void* dout,
                           const float* saved, int ci, float* ws, void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, int64_t T_,
                           int D, const ScanOpts& opt, float* dbias, hipStream_t s) {
    const ScanWs L = scan_ws_layout(T_, D, NS, ci);
    const int lc = bwd_chunk_len(T_, D, NS);
    const int64_t nchunk = (T_ + lc - 1) / lc;
    const int ls = bwd_sum_len(T_, D, NS);  // summary sub-chunk: lc = 2^logR ls
    const int logR = __builtin_ctz((unsigned)(lc / ls));
    const dim3 grid((unsigned)(L.ngroup * L.nsum));  // summary kernel: 64 channels per wave
    const int64_t ND = (int64_t)NS * D;
    const int vec = stage_vec_ok<T>(D, {u, delta, z, dout}) ? 1 : 0;
    k_bc_to_f32<T, NS><<<(unsigned)((T_ * 2 * NS + 255) / 256), 256, 0, s>>>((const T*)B, (const T*)C, ws + L.bc,
                                                                            T_);
    SSMP_LAUNCH_CHECK();
    // the state entering every kCK-th token: kept by the forward, or replayed
    const float* ckpt = saved;
    int ckshift = ci ? __builtin_ctz((unsigned)ci) : 0;
    if (!ck_direct(ci)) {
        ckshift = __builtin_ctz((unsigned)kCK);
        const int st = scan_dense_ckpt(NS, std::is_same<T, uint16_t>::value, u, delta, A, pos, saved, ci, ws, T_, D,
                                       opt, s);
        if (st) return st;
        ckpt = ws + L.dense;
    }
    if (L.nsum > 1) {
        if (z)
            k_scan_bwd_summary<T, NS, true><<<grid, kWave, 0, s>>>((const T*)delta, A, ws + L.bc, (const T*)z,
                                                                   (const T*)dout, pos, ws + L.Pr, ws + L.Sr, T_, D,
                                                                   vec, ls, logR, opt);
        else
            k_scan_bwd_summary<T, NS, false><<<grid, kWave, 0, s>>>((const T*)delta, A, ws + L.bc, nullptr,
                                                                    (const T*)dout, pos, ws + L.Pr, ws + L.Sr, T_, D,
                                                                    vec, ls, logR, opt);
        SSMP_LAUNCH_CHECK();
    }
    k_scan_bwd_carry<NS><<<(unsigned)((ND + 255) / 256), 256, 0, s>>>(ws + L.Pr, ws + L.Sr, A, pos, ws + L.cin,
                                                                      D, L.nsum, ls, logR);
    SSMP_LAUNCH_CHECK();
    BwdArgs<T> a;
    a.u = (const T*)u; a.delta = (const T*)delta; a.A = A; a.bc = ws + L.bc; a.Dskip = Dskip;
    a.z = (const T*)z; a.dout = (const T*)dout; a.pos = pos; a.ckpt = ckpt; a.ckshift = ckshift; a.cin = ws + L.cin;
    a.du = (T*)du; a.ddelta = (T*)ddelta; a.dz = (T*)dz; a.dApart = ws + L.dApart; a.dDpart = ws + L.dDpart;
    a.dbpart = ws + L.dbpart; a.dBC = ws + L.dBC; a.sink = ws + L.sink; a.T_ = T_; a.D = D; a.lc = lc; a.opt = opt;
    constexpr int SW = Split<NS>::SW;
    const int64_t ngroup = (D + kGroupCh - 1) / kGroupCh;
    const dim3 mgrid((unsigned)(ngroup * nchunk));
    const bool xs = opt.delta_bias != nullptr || opt.softplus != 0;
    // sequence states get kernels of their own, so the reset-only ones keep
    // their register allocation
    const bool st = opt.h0 != nullptr || opt.dhT != nullptr || opt.dh0 != nullptr;
#define SSMP_BWD_MAIN(G, X, S) k_scan_bwd_main<T, NS, G, X, S><<<mgrid, kWave * SW, 0, s>>>(a, ws + L.bc)
#define SSMP_BWD_MAIN_S(G, X)               \
    if (st) SSMP_BWD_MAIN(G, X, true);      \
    else SSMP_BWD_MAIN(G, X, false)
    if (z) {
        if (xs) { SSMP_BWD_MAIN_S(true, true); } else { SSMP_BWD_MAIN_S(true, false); }
    } else {
        if (xs) { SSMP_BWD_MAIN_S(false, true); } else { SSMP_BWD_MAIN_S(false, false); }
    }
#undef SSMP_BWD_MAIN_S
#undef SSMP_BWD_MAIN
    SSMP_LAUNCH_CHECK();
    const int64_t nrp = ND > D ? ND : D;
    k_scan_bwd_reduce_params<NS><<<(unsigned)((nrp + 255) / 256), 256, 0, s>>>(
        ws + L.dApart, ws + L.dDpart, ws + L.dbpart, nchunk, D, dA, dD, xs ? dbias : nullptr);
    SSMP_LAUNCH_CHECK();
    k_scan_bwd_reduce_bc<NS><<<(unsigned)((T_ * 2 * NS + 255) / 256), 256, 0, s>>>(ws + L.dBC, ngroup, T_, dB, dC);
    SSMP_LAUNCH_CHECK();
    if (opt.dh0) {
        const int64_t n = (int64_t)opt.nseq * ND;
        k_empty_seq_states<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(opt.cu, opt.nseq, ND, opt.dhT, opt.dh0);
        SSMP_LAUNCH_CHECK();
    }
    return SSMP_OK;
}

template <typename T>
static int scan_bwd_dispatch(int N, const void* u, const void* delta, const float* A, const void* B, const void* C,
                             const float* Dskip, const void* z, const int32_t* pos, const void* dout,
                             const float* saved, int ci, float* ws, void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                             int64_t T_, int D, const ScanOpts& o, float* dbias, hipStream_t s) {
#define SSMP_BWD_CASE(NV)                                                                                         \
    case NV:                                                                                                      \
        return scan_bwd_launch<T, NV>(u, delta, A, B, C, Dskip, z, pos, dout, saved, ci, ws, du, ddelta, dA, dB,   \
                                      dC, dD, dz, T_, D, o, dbias, s);
    switch (N) {
        SSMP_BWD_CASE(1)
        SSMP_BWD_CASE(2)
        SSMP_BWD_CASE(4)
        SSMP_BWD_CASE(8)
        SSMP_BWD_CASE(16)
        default: return SSMP_ERR_UNSUPPORTED;
    }
#undef SSMP_BWD_CASE
}

}  // namespace ssmp

extern "C" int selective_scan_pack_bwd_ck(const void* u, const void* delta, const float* A, const void* B,
                                          const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                          const void* dout, void* du, void* ddelta, float* dA, float* dB, float* dC,
                                          float* dD, void* dz, int64_t T, int32_t D, int32_t N, int32_t dtype,
                                          const float* delta_bias, int32_t delta_softplus, float gate_floor,
                                          float* ddelta_bias, const int32_t* cu_seqlens, int32_t nseq,
                                          const float* initial_state, const float* dfinal_state,
                                          float* dinitial_state, int32_t ckpt_interval, const void* saved,
                                          size_t saved_bytes, void* scratch, size_t scratch_bytes, void* stream) {
    using namespace ssmp;
    int st = scan_check_args(T, D, N, dtype);
    if (st) return st;
    if (!ck_interval_ok(ckpt_interval)) return SSMP_ERR_SHAPE;
    if (!A || !dA) return SSMP_ERR_NULL;
    if ((Dskip == nullptr) != (dD == nullptr)) return SSMP_ERR_NULL;
    if ((z == nullptr) != (dz == nullptr)) return SSMP_ERR_NULL;
    if ((delta_bias == nullptr) != (ddelta_bias == nullptr)) return SSMP_ERR_NULL;
    const bool states = initial_state || dfinal_state || dinitial_state;
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
        o.dhT = dfinal_state;
        o.dh0 = dinitial_state;
    }
    if (T == 0) {
        // empty input: the sums are zero, and every sequence hands its
        // final-state gradient back unchanged
        if ((st = zero_f32(dA, (int64_t)D * N, s))) return st;
        if ((st = zero_f32(dD, D, s))) return st;
        if ((st = zero_f32(ddelta_bias, D, s))) return st;
        if (!dinitial_state) return SSMP_OK;
        const int64_t ND = (int64_t)D * N, n = (int64_t)nseq * ND;
        k_empty_seq_states<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(cu_seqlens, nseq, ND, dfinal_state,
                                                                       dinitial_state);
        return hipGetLastError() == hipSuccess ? SSMP_OK : SSMP_ERR_HIP;
    }
    if (!u || !delta || !B || !C || !pos || !dout || !du || !ddelta || !dB || !dC) return SSMP_ERR_NULL;
    if (ckpt_interval && (!saved || saved_bytes < selective_scan_pack_saved_bytes(T, D, N, ckpt_interval)))
        return SSMP_ERR_WORKSPACE;
    if (!scratch || scratch_bytes < selective_scan_pack_bwd_scratch_bytes(T, D, N, ckpt_interval))
        return SSMP_ERR_WORKSPACE;
    const float* sv = ckpt_interval ? static_cast<const float*>(saved) : nullptr;
    float* ws = static_cast<float*>(scratch);
    return dtype == SSMP_BF16
               ? scan_bwd_dispatch<uint16_t>(N, u, delta, A, B, C, Dskip, z, pos, dout, sv, ckpt_interval, ws, du,
                                             ddelta, dA, dB, dC, dD, dz, T, D, o, ddelta_bias, s)
               : scan_bwd_dispatch<float>(N, u, delta, A, B, C, Dskip, z, pos, dout, sv, ckpt_interval, ws, du,
                                          ddelta, dA, dB, dC, dD, dz, T, D, o, ddelta_bias, s);
}

extern "C" int selective_scan_pack_bwd_states(const void* u, const void* delta, const float* A, const void* B,
                                              const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                              const void* dout, void* workspace, size_t workspace_bytes, void* du,
                                              void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                                              int64_t T, int32_t D, int32_t N, int32_t dtype,
                                              const float* delta_bias, int32_t delta_softplus, float gate_floor,
                                              float* ddelta_bias, const int32_t* cu_seqlens, int32_t nseq,
                                              const float* initial_state, const float* dfinal_state,
                                              float* dinitial_state, void* stream) {
    // the workspace: the forward's checkpoints every kCK tokens, then the
    // scratch (a short one is passed on as none, so that the argument checks
    // come first)
    const size_t sb = selective_scan_pack_saved_bytes(T, D, N, ssmp::kCK);
    const bool ok = workspace && workspace_bytes >= selective_scan_pack_workspace_bytes(T, D, N);
    char* w = ok ? static_cast<char*>(workspace) : nullptr;
    return selective_scan_pack_bwd_ck(u, delta, A, B, C, Dskip, z, pos, dout, du, ddelta, dA, dB, dC, dD, dz, T, D,
                                      N, dtype, delta_bias, delta_softplus, gate_floor, ddelta_bias, cu_seqlens,
                                      nseq, initial_state, dfinal_state, dinitial_state, ssmp::kCK, w, ok ? sb : 0,
                                      w ? w + sb : nullptr, ok ? workspace_bytes - sb : 0, stream);
}

extern "C" int selective_scan_pack_bwd_ex(const void* u, const void* delta, const float* A, const void* B,
                                          const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                          const void* dout, void* workspace, size_t workspace_bytes, void* du,
                                          void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                                          int64_t T, int32_t D, int32_t N, int32_t dtype, const float* delta_bias,
                                          int32_t delta_softplus, float gate_floor, float* ddelta_bias,
                                          void* stream) {
    return selective_scan_pack_bwd_states(u, delta, A, B, C, Dskip, z, pos, dout, workspace, workspace_bytes, du,
                                          ddelta, dA, dB, dC, dD, dz, T, D, N, dtype, delta_bias, delta_softplus,
                                          gate_floor, ddelta_bias, nullptr, 0, nullptr, nullptr, nullptr, stream);
}

extern "C" int selective_scan_pack_bwd(const void* u, const void* delta, const float* A, const void* B,
                                       const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                       const void* dout, void* workspace, size_t workspace_bytes, void* du,
                                       void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                                       int64_t T, int32_t D, int32_t N, int32_t dtype, void* stream) {
    return selective_scan_pack_bwd_ex(u, delta, A, B, C, Dskip, z, pos, dout, workspace, workspace_bytes, du, ddelta,
                                      dA, dB, dC, dD, dz, T, D, N, dtype, nullptr, 0, 0.0f, nullptr, stream);
}
