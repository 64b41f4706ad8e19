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
// kBB-token blocks (inputs staged through LDS, the next block in flight); each
// kK-token sub-chunk restarts from the forward's checkpoint at its first token
// and replays its tokens with their states held in VGPRs before running the
// reverse step over them. dB and dC (sums over channels) are reduced
// across each wave and then across the workgroup's waves through LDS, and
// written per workgroup channel group; dA and dDskip
// are written per chunk; small kernels finish both sums in a fixed order, so
// results are deterministic.
#include "scan_common.h"

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
        if (more) {
#pragma unroll
            for (int n = 0; n < NS; ++n) nxt[n] = rows[(k + 1) * 2 * NS + n];
        }
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
                                                         int D, int vec, int lc, ScanOpts opt) {
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
    if (c == 0) return;            // nothing to the left
    if (pos[t0] == 0) return;      // starts at a head: carries nothing out

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
        int32_t hp;  // pos at the start of chunk cb - lane (lanes < kB, chunks >= 1)
    };
    const int dch = (int)(i % D);
    const float A2 = A[(size_t)dch * NS + (int)(i / D)] * kLog2e;
    auto load = [&](Batch& b, int64_t cb) {
        const int64_t cj = cb - lane;
        b.hp = (lane < kB && cj >= 1) ? pos[cj * lc] : 1;
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
        const uint64_t heads = __ballot(cur.hp == 0);  // bit j: chunk cb - j >= 1 starts at a head
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            const int64_t c = cb - j;
            if (c >= 0 && (((c + 1) & rmask) == 0 || c == nchunk - 1)) {
                if (act) *cp = cc;
                cp -= ND;
            }
            // select at heads, as in the forward
            const float tj = cur.P[j];
            const float Pj = (tj != tj) ? 0.0f : exp2_fast(A2 * tj);
            const float cn = ((heads >> j) & 1u) ? 0.0f : (Pj == 0.0f) ? cur.S[j] : __builtin_fmaf(Pj, cc, cur.S[j]);
            cc = (c >= 1) ? cn : cc;
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
    const float* ckpt;
    const float* cin;
    T* du;
    T* ddelta;
    T* dz;
    float* dApart;
    float* dDpart;
    float* dbpart;
    float* dBC;
    int64_t T_;
    int D;
    int vec;
    int lc;
    ScanOpts opt;
};

constexpr int kRedStride = kWave + 4;  // LDS row stride (floats) of the dB/dC transpose

// The decays a = exp2(delta A2) of a sub-chunk's replay are kept for its
// reverse step (32 VGPRs at d_state 16) where the registers allow: with 2-byte
// inputs the backward's main kernel fits them without spilling, with fp32
// inputs (larger staging) it would spill, so it computes them again.
template <typename T>
constexpr bool kCacheDecay = sizeof(T) == 2;

// Replay of one kK-token sub-chunk from its entering state h: the states hh[k]
// after each token, their decays ak[k] (kCacheDecay) and the pre-gate outputs
// yk[k]. SAFE sub-chunks may be
// short (ns < kK) and may hold heads; the fast ones are full and head-free.
// With initial states, a head starts from its sequence's h0 (this lane's
// share of the states) instead of zero.
template <bool SAFE, bool XS, bool ST, int NS, int LPC, typename St, typename T>
__device__ __forceinline__ void bwd_replay(const T* lds, const float* bcl, int kb, int ns, uint32_t heads, int ch,
                                           int n0, const float (&A2)[NS / LPC], float (&h)[NS / LPC],
                                           float (&hh)[kK][NS / LPC], float (&ak)[kK][NS / LPC], float (&yk)[kK],
                                           float (&dtk)[kK], float (&slk)[kK], float Dv, const StepMap& sm,
                                           const ScanOpts& opt, int64_t tb, int D, int dd) {
    // on return h holds the state after the last replayed token
    constexpr int NH = NS / LPC;
    if constexpr (XS) {
        // mapped steps and their slopes for the whole sub-chunk (past ns the
        // staged rows are stale and the results unused). A lane pair shares
        // its channel: each lane maps every other token and the pair swaps.
        if constexpr (LPC == 2) {
            static_assert(kK % 2 == 0, "tokens come in pairs");
            const bool odd = n0 != 0;
#pragma unroll
            for (int j = 0; j < kK / 2; ++j) {
                float sl_own;
                const float dt_own = sm.eff(St::get(lds, 1, kb + 2 * j + (odd ? 1 : 0), ch), sl_own);
                const float dt_oth = swap_adjacent(dt_own), sl_oth = swap_adjacent(sl_own);
                dtk[2 * j] = odd ? dt_oth : dt_own;
                dtk[2 * j + 1] = odd ? dt_own : dt_oth;
                slk[2 * j] = odd ? sl_oth : sl_own;
                slk[2 * j + 1] = odd ? sl_own : sl_oth;
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < kK; ++kk) dtk[kk] = sm.eff(St::get(lds, 1, kb + kk, ch), slk[kk]);
        }
    }
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
        if constexpr (SAFE) {
            if (kk >= ns) break;
        }
        const int k = kb + kk;
        const float dt = XS ? dtk[kk] : St::get(lds, 1, k, ch);
        const float uu = St::get(lds, 0, k, ch);
        const float dtu = dt * uu;
        const float* row = bcl + k * 2 * NS + n0;
        if constexpr (SAFE) {
            if ((heads >> k) & 1u) {
                asm volatile("");
                if (ST && opt.h0) {
                    const float* __restrict__ hp =
                        opt.h0 + ((size_t)seq_of(opt.cu, opt.nseq, tb + k) * D + dd) * NS + n0;
#pragma unroll
                    for (int i = 0; i < NH; ++i) h[i] = hp[i];
                } else {
#pragma unroll
                    for (int i = 0; i < NH; ++i) h[i] = 0.0f;
                }
            }
        }
        float y = 0.0f;
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const float a = exp2_fast(dt * A2[i]);
            if constexpr (kCacheDecay<T>) ak[kk][i] = a;
            h[i] = __builtin_fmaf(a, h[i], dtu * row[i]);
            hh[kk][i] = h[i];
            y = __builtin_fmaf(row[NS + i], h[i], y);
        }
        if constexpr (LPC == 2) y += swap_adjacent(y);
        yk[kk] = __builtin_fmaf(Dv, uu, y);
    }
}

// Per-block outputs: du, ddelta, dz rows (dtype T) and the wave's per-token
// dB/dC sums (LDS, [kBB][2NS]).
template <typename T>
struct BwdRows {
    T* du;
    T* ddelta;
    T* dz;
    float* dbc;
};

// Reverse step over one sub-chunk (tokens kb + ns - 1 down to kb).
template <bool SAFE, bool GATE, bool XS, bool ST, int NS, int LPC, typename St, typename T>
__device__ __forceinline__ void bwd_reverse(const T* lds, const float* bcl, float (*red)[kRedStride], int kb, int ns,
                                            uint32_t heads, int lane, int ch, int sh, int n0, bool act, bool full,
                                            int D, int d, const float (&A2)[NS / LPC], float (&carry)[NS / LPC],
                                            float (&dA)[NS / LPC], float& dDacc, float Dv,
                                            const float (&hin)[NS / LPC], const float (&hh)[kK][NS / LPC],
                                            const float (&ak)[kK][NS / LPC],
                                            const float (&yk)[kK], const float (&dtk)[kK], const float (&slk)[kK],
                                            const BwdRows<T>& rows, float gf, float& dbacc, const ScanOpts& opt,
                                            int64_t tb, int dd) {
    constexpr int NH = NS / LPC;
    constexpr int CW = kWave / LPC;
#pragma unroll
    for (int kk = kK - 1; kk >= 0; --kk) {
        if constexpr (SAFE) {
            if (kk >= ns) continue;
        }
        const int k = kb + kk;
        const float dt = XS ? dtk[kk] : St::get(lds, 1, k, ch);
        const float uu = St::get(lds, 0, k, ch);
        const float go = St::get(lds, 3, k, ch);
        float gg = go, dzv = 0.0f;
        if constexpr (GATE) {
            const float zz = St::get(lds, 2, k, ch);
            const float sg = sigmoid_fast(zz);
            gg = go * __builtin_fmaf(zz, sg, gf);
            dzv = go * yk[kk] * sg * (1.0f + zz * (1.0f - sg));
        }
        gg = act ? gg : 0.0f;  // lanes past D add nothing to dB/dC
        const float dtu = act ? dt * uu : 0.0f;
        const float* row = bcl + k * 2 * NS + n0;
        const int col = sh * CW + ch;
        float sumB = 0.0f, sumAr = 0.0f;
        const bool head = SAFE && ((heads >> k) & 1u);
        if (head) {
            asm volatile("");
            // With states, what the decay passes back out of the head is the
            // initial state's gradient, the initial state is the previous
            // state of the r term, and the carry into the token before the
            // head (the previous sequence's last) is that sequence's
            // final-state gradient.
            const bool st = ST && (opt.h0 || opt.dh0);
            const int64_t t = tb + k;
            const size_t so = st ? ((size_t)seq_of(opt.cu, opt.nseq, t) * D + dd) * NS + n0 : 0;
            const float* __restrict__ gp = (ST && opt.dhT && t > 0)
                                               ? opt.dhT + ((size_t)seq_of(opt.cu, opt.nseq, t - 1) * D + dd) * NS + n0
                                               : nullptr;
#pragma unroll
            for (int i = 0; i < NH; ++i) {
                const float dh = __builtin_fmaf(gg, row[NS + i], carry[i]);
                red[i][col] = dh * dtu;             // dB row
                red[NH + i][col] = gg * hh[kk][i];  // dC row
                sumB = __builtin_fmaf(dh, row[i], sumB);
                if (st) {
                    const float cr = (kCacheDecay<T> ? ak[kk][i] : exp2_fast(dt * A2[i])) * dh;
                    if (opt.h0) {
                        const float r = cr * opt.h0[so + i];
                        sumAr = __builtin_fmaf(r, A2[i], sumAr);
                        dA[i] = __builtin_fmaf(r, dt, dA[i]);
                    }
                    if (opt.dh0 && act) opt.dh0[so + i] = cr;
                }
                carry[i] = (gp && act) ? gp[i] : 0.0f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NH; ++i) {
                const float dh = __builtin_fmaf(gg, row[NS + i], carry[i]);
                red[i][col] = dh * dtu;
                red[NH + i][col] = gg * hh[kk][i];
                sumB = __builtin_fmaf(dh, row[i], sumB);
                // carry to t-1: a_t dh_t; r = dh_t a_t h_{t-1}
                carry[i] = (kCacheDecay<T> ? ak[kk][i] : exp2_fast(dt * A2[i])) * dh;
                const float r = carry[i] * (kk == 0 ? hin[i] : hh[kk > 0 ? kk - 1 : 0][i]);
                sumAr = __builtin_fmaf(r, A2[i], sumAr);
                dA[i] = __builtin_fmaf(r, dt, dA[i]);
            }
        }
        if constexpr (LPC == 2) {
            sumB += swap_adjacent(sumB);
            sumAr += swap_adjacent(sumAr);
        }
        const float duv = __builtin_fmaf(gg, Dv, dt * sumB);
        float ddv = __builtin_fmaf(uu, sumB, sumAr * kLn2);
        if constexpr (XS) {
            ddv *= slk[kk];  // with respect to the stored step
            dbacc += act ? ddv : 0.0f;
        }
        dDacc = __builtin_fmaf(gg, uu, dDacc);
        // both lanes of a pair hold the same values and store the same bytes
        const uint32_t e = (uint32_t)(k * D + d);  // < kBB * D, fits 32 bits
        if (full || act) {
            Elt<T>::st(rows.du, e, duv);
            Elt<T>::st(rows.ddelta, e, ddv);
            if constexpr (GATE) Elt<T>::st(rows.dz, e, dzv);
        }
        // dB/dC of state n: the sum of row (n % NH) (dB) or NH + n % NH (dC)
        // over the columns of share n / NH. Two lanes per output value, each
        // adding half the columns; both then hold the total.
        wave_sync();
        const int o = lane >> 1, hf = lane & 1;  // output o: kind o / NS, state o % NS
        constexpr bool all_out = 4 * NS >= kWave;
        float v = 0.0f;
        if (all_out || o < 2 * NS) {
            const int kind = o / NS, n = o % NS;
            const int rrow = kind * NH + (n % NH);
            const int c0 = (n / NH) * CW + hf * (CW / 2);
            const float4* rw = reinterpret_cast<const float4*>(&red[rrow][c0]);
            float4 r4 = rw[0];
            v = (r4.x + r4.y) + (r4.z + r4.w);
#pragma unroll
            for (int q = 1; q < CW / 8; ++q) {
                r4 = rw[q];
                v += (r4.x + r4.y) + (r4.z + r4.w);
            }
        }
        v += swap_adjacent(v);
        if (all_out || o < 2 * NS) rows.dbc[(uint32_t)(k * 2 * NS + o)] = v;
        wave_sync();
    }
}

// LPC lanes share a channel, each holding NS/LPC of its states, so a wave
// covers 64/LPC channels. Two lanes per channel halve the registers and LDS a
// wave needs, which lets two or more waves share a SIMD; per-channel sums over
// the states are completed with one DPP exchange between the lane pair.
// A workgroup holds WV waves on adjacent channel groups of one chunk: they
// share the staged B/C rows of each block, and add their per-token dB/dC sums
// in LDS, so one partial row per WV*64/LPC channels reaches memory.
template <typename T, int NS, int LPC, int WV, bool GATE, bool XS, bool ST>
__global__ __launch_bounds__(kWave * WV, 2) void k_scan_bwd_main(BwdArgs<T> p) {
    constexpr int NH = NS / LPC;      // states per lane
    constexpr int CW = kWave / LPC;   // channels per wave
    static_assert(NH * LPC == NS && (LPC == 1 || LPC == 2), "lane split");
    static_assert(CW * WV >= kWave, "dB/dC partial rows are sized for groups of at least 64 channels");
    using St = Stager<T, 4, kBB, CW>;  // u, delta, z, dout
    constexpr int NT = kWave * WV;     // threads
    constexpr int BCW = 2 * NS;        // dB/dC values per token
    __shared__ __attribute__((aligned(16))) T lds[WV][St::kElems];
    __shared__ __attribute__((aligned(16))) float bcl[kBB * BCW];  // B/C rows of the block
    __shared__ __attribute__((aligned(16))) float red[WV][2 * NH][kRedStride];
    __shared__ float blk[WV][kBB * BCW];  // per-wave dB/dC sums of the block's tokens

    const int tid = threadIdx.x;
    const int wv = tid / kWave;
    const int lane = tid % kWave;
    const int ch = lane / LPC;        // channel within the wave's group
    const int sh = lane % LPC;        // which share of the states
    const Tile tl = tile_of_w<CW * WV>(p.D);
    const int gw = tl.g;              // workgroup channel group
    const int g = gw * WV + wv;       // wave channel group
    const int d = g * CW + ch;
    const bool act = d < p.D;
    const bool full = (g + 1) * CW <= p.D;
    const int dd = act ? d : p.D - 1;
    const int64_t c = tl.c;
    const int64_t t0 = c * p.lc;
    const int64_t t1 = (t0 + p.lc < p.T_) ? t0 + p.lc : p.T_;
    const size_t ND = (size_t)NS * p.D;
    const int n0 = sh * NH;           // first state of this lane
    const int D = p.D;
    T* const mylds = lds[wv];

    // lanes past D carry zeros throughout, so they add nothing to dB/dC
    float A2[NH], carry[NH], dA[NH];
#pragma unroll
    for (int i = 0; i < NH; ++i) {
        A2[i] = p.A[(size_t)dd * NS + n0 + i] * kLog2e;
        carry[i] = act ? p.cin[(size_t)c * ND + (size_t)(n0 + i) * D + dd] : 0.0f;
        dA[i] = 0.0f;
    }
    if (ST && p.opt.dhT && act && (t1 == p.T_ || p.pos[t1] == 0)) {
        // the chunk ends at a sequence's last token (the carry pass hands it
        // zero): it starts from that sequence's final-state gradient
        const float* __restrict__ gp = p.opt.dhT + ((size_t)seq_of(p.opt.cu, p.opt.nseq, t1 - 1) * D + dd) * NS + n0;
#pragma unroll
        for (int i = 0; i < NH; ++i) carry[i] = gp[i];
    }
    const float Dv = (p.Dskip && act) ? p.Dskip[dd] : 0.0f;
    float dDacc = 0.0f, dbacc = 0.0f;
    const StepMap sm = step_map(p.opt, dd);
    const float gf = p.opt.gate_floor;
    const T* const src[4] = {p.u, p.delta, GATE ? p.z : p.u, p.dout};

    // B/C rows of a block: kBB * 2NS floats, fetched with the block's inputs
    // by the first BCV threads of the workgroup
    constexpr int BCV = kBB * BCW / 4;                    // float4 pieces
    constexpr int BCP = (BCV + NT - 1) / NT;              // pieces per thread
    float4 bcr[BCP];
    auto fetch_bc = [&](int64_t tb) {
        const float* srcf = p.bc + (size_t)tb * BCW;  // 16-byte aligned: tb is a multiple of kBB
        const float4* srcv = reinterpret_cast<const float4*>(srcf);
        // floats of the block's rows inside the tensor; with 2N not a multiple
        // of 4 the last piece can be partial, and is read float by float
        const int lim = (int)((p.T_ - tb < kBB) ? (p.T_ - tb) : kBB) * BCW;
#pragma unroll
        for (int q = 0; q < BCP; ++q) {
            const int idx = q * NT + tid;
            const int f0 = idx * 4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (idx < BCV && f0 + 4 <= lim) {
                v = srcv[idx];
            } else if (idx < BCV && f0 < lim) {
                v.x = srcf[f0];
                if (f0 + 1 < lim) v.y = srcf[f0 + 1];
                if (f0 + 2 < lim) v.z = srcf[f0 + 2];
            }
            bcr[q] = v;
        }
    };
    auto commit_bc = [&]() {
#pragma unroll
        for (int q = 0; q < BCP; ++q) {
            const int idx = q * NT + tid;
            if (idx < BCV) reinterpret_cast<float4*>(bcl)[idx] = bcr[q];
        }
    };

    // Each sub-chunk restarts from the checkpoint at its first token; the
    // next sub-chunk's state (kK tokens earlier) is loaded while this one runs.
    auto load_state = [&](int64_t ts, float (&hs)[NH]) {
        ck_load<NS, NH>(p.ckpt + (size_t)(ts / kCK) * ND, dd, D, n0, act, hs);
    };

    const int64_t nblk = (t1 - t0 + kBB - 1) / kBB;
    St st;
    float hn[NH];
    {
        const int64_t tl0 = t0 + (nblk - 1) * kBB;
        st.fetch(src, tl0, p.T_, D, g, lane, p.vec);
        fetch_bc(tl0);
        load_state(tl0 + ((t1 - tl0 - 1) / kK) * kK, hn);  // last sub-chunk of the chunk
    }
    for (int64_t jb = nblk - 1; jb >= 0; --jb) {
        const int64_t tb0 = t0 + jb * kBB;
        const int nb = (int)(((tb0 + kBB < t1) ? tb0 + kBB : t1) - tb0);  // tokens in this block
        const int nsub = (nb + kK - 1) / kK;
        const uint32_t heads = block_heads<kBB>(p.pos, tb0, p.T_, lane);
        __syncthreads();  // every wave is done with the previous block's bcl and blk
        st.commit(mylds, src, tb0, p.T_, D, g, lane, p.vec);
        commit_bc();
        __syncthreads();
        if (jb > 0) {
            st.fetch(src, tb0 - kBB, p.T_, D, g, lane, p.vec);
            fetch_bc(tb0 - kBB);
        }
        const BwdRows<T> rows{p.du + (size_t)tb0 * D, p.ddelta + (size_t)tb0 * D,
                              GATE ? p.dz + (size_t)tb0 * D : nullptr, blk[wv]};

        for (int sc = nsub - 1; sc >= 0; --sc) {
            const int kb = sc * kK;  // first token of the sub-chunk within the block
            const int ns = (nb - kb < kK) ? nb - kb : kK;
            float h[NH], hin[NH], hh[kK][NH], ak[kK][NH], yk[kK], dtk[kK], slk[kK];
#pragma unroll
            for (int i = 0; i < NH; ++i) {
                h[i] = hn[i];
                hin[i] = hn[i];
            }
            if (tb0 + kb - kK >= t0) load_state(tb0 + kb - kK, hn);
            const uint32_t sub_heads = (heads >> kb) & ((1u << kK) - 1u);
            if (sub_heads == 0 && ns == kK) {
                bwd_replay<false, XS, ST, NS, LPC, St>(mylds, bcl, kb, kK, 0u, ch, n0, A2, h, hh, ak, yk, dtk, slk, Dv,
                                                       sm, p.opt, tb0, D, dd);
                bwd_reverse<false, GATE, XS, ST, NS, LPC, St>(mylds, bcl, red[wv], kb, kK, 0u, lane, ch, sh, n0, act,
                                                              full, D, d, A2, carry, dA, dDacc, Dv, hin, hh, ak, yk,
                                                              dtk, slk, rows, gf, dbacc, p.opt, tb0, dd);
            } else {
                bwd_replay<true, XS, ST, NS, LPC, St>(mylds, bcl, kb, ns, heads, ch, n0, A2, h, hh, ak, yk, dtk, slk,
                                                      Dv, sm, p.opt, tb0, D, dd);
                bwd_reverse<true, GATE, XS, ST, NS, LPC, St>(mylds, bcl, red[wv], kb, ns, heads, lane, ch, sh, n0, act,
                                                             full, D, d, A2, carry, dA, dDacc, Dv, hin, hh, ak, yk,
                                                             dtk, slk, rows, gf, dbacc, p.opt, tb0, dd);
            }
        }

        // the workgroup's dB/dC sums of the block, waves added in order
        __syncthreads();
        float* const dst = p.dBC + ((size_t)gw * p.T_ + tb0) * BCW;
        for (int e = tid; e < nb * BCW; e += NT) {
            float v = blk[0][e];
#pragma unroll
            for (int w = 1; w < WV; ++w) v += blk[w][e];
            dst[e] = v;
        }
    }
    if (act) {
#pragma unroll
        for (int i = 0; i < NH; ++i) p.dApart[(size_t)c * ND + (size_t)(n0 + i) * D + d] = dA[i];
        if (sh == 0) p.dDpart[(size_t)c * D + d] = dDacc;
        if (XS && sh == 0) p.dbpart[(size_t)c * D + d] = dbacc;
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
                           const float* Dskip, const void* z, const int32_t* pos, const void* dout, float* ws,
                           void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, int64_t T_,
                           int D, const ScanOpts& opt, float* dbias, hipStream_t s) {
    const ScanWs L = scan_ws_layout(T_, D, NS);
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
    if (L.nsum > 1) {
        if (z)
            k_scan_bwd_summary<T, NS, true><<<grid, kWave, 0, s>>>((const T*)delta, A, ws + L.bc, (const T*)z,
                                                                   (const T*)dout, pos, ws + L.Pr, ws + L.Sr, T_, D,
                                                                   vec, ls, opt);
        else
            k_scan_bwd_summary<T, NS, false><<<grid, kWave, 0, s>>>((const T*)delta, A, ws + L.bc, nullptr,
                                                                    (const T*)dout, pos, ws + L.Pr, ws + L.Sr, T_, D,
                                                                    vec, ls, opt);
        SSMP_LAUNCH_CHECK();
    }
    k_scan_bwd_carry<NS><<<(unsigned)((ND + 255) / 256), 256, 0, s>>>(ws + L.Pr, ws + L.Sr, A, pos, ws + L.cin,
                                                                      D, L.nsum, ls, logR);
    SSMP_LAUNCH_CHECK();
    BwdArgs<T> a;
    a.u = (const T*)u; a.delta = (const T*)delta; a.A = A; a.bc = ws + L.bc; a.Dskip = Dskip;
    a.z = (const T*)z; a.dout = (const T*)dout; a.pos = pos; a.ckpt = ws + L.ckpt; a.cin = ws + L.cin;
    a.du = (T*)du; a.ddelta = (T*)ddelta; a.dz = (T*)dz; a.dApart = ws + L.dApart; a.dDpart = ws + L.dDpart;
    a.dbpart = ws + L.dbpart; a.dBC = ws + L.dBC; a.T_ = T_; a.D = D; a.vec = vec; a.lc = lc; a.opt = opt;
    constexpr int LPC = NS >= 4 ? 2 : 1;  // bwd_lanes_per_channel
    constexpr int WV = bwd_waves_per_group(sizeof(T));
    const int64_t ngroup = bwd_bc_groups(D, NS, sizeof(T));
    const dim3 mgrid((unsigned)(ngroup * nchunk));
    const bool xs = opt.delta_bias != nullptr || opt.softplus != 0;
    // sequence states get kernels of their own, so the reset-only ones keep
    // their register allocation
    const bool st = opt.h0 != nullptr || opt.dhT != nullptr || opt.dh0 != nullptr;
#define SSMP_BWD_MAIN(G, X, S) k_scan_bwd_main<T, NS, LPC, WV, G, X, S><<<mgrid, kWave * WV, 0, s>>>(a)
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
                             const float* Dskip, const void* z, const int32_t* pos, const void* dout, float* ws,
                             void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                             int64_t T_, int D, const ScanOpts& o, float* dbias, hipStream_t s) {
#define SSMP_BWD_CASE(NV)                                                                                         \
    case NV:                                                                                                      \
        return scan_bwd_launch<T, NV>(u, delta, A, B, C, Dskip, z, pos, dout, ws, du, ddelta, dA, dB, dC, dD, dz, \
                                      T_, D, o, dbias, s);
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

extern "C" int selective_scan_pack_bwd_states(const void* u, const void* delta, const float* A, const void* B,
                                              const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                              const void* dout, void* workspace, size_t workspace_bytes, void* du,
                                              void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                                              int64_t T, int32_t D, int32_t N, int32_t dtype,
                                              const float* delta_bias, int32_t delta_softplus, float gate_floor,
                                              float* ddelta_bias, const int32_t* cu_seqlens, int32_t nseq,
                                              const float* initial_state, const float* dfinal_state,
                                              float* dinitial_state, void* stream) {
    using namespace ssmp;
    int st = scan_check_args(T, D, N, dtype);
    if (st) return st;
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
    if (!workspace || workspace_bytes < selective_scan_pack_workspace_bytes(T, D, N)) return SSMP_ERR_WORKSPACE;
    float* ws = static_cast<float*>(workspace);
    return dtype == SSMP_BF16 ? scan_bwd_dispatch<uint16_t>(N, u, delta, A, B, C, Dskip, z, pos, dout, ws, du,
                                                            ddelta, dA, dB, dC, dD, dz, T, D, o, ddelta_bias, s)
                              : scan_bwd_dispatch<float>(N, u, delta, A, B, C, Dskip, z, pos, dout, ws, du, ddelta,
                                                         dA, dB, dC, dD, dz, T, D, o, ddelta_bias, s);
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
