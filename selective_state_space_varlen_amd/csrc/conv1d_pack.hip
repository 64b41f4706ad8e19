// conv1d_pack forward and backward: causal depthwise conv of width W <= 4 that
// stops at each sequence's head token.
//
// Shanghai AI Lab article on packed variable-length Mamba-1 training
// (gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), section "conv1d_pack 算子":
// the conv looks back W-1 tokens and terminates early at a head; the backward
// stops dx and dweight the same way, taking the reverse position from the
// position index W-1 tokens ahead.
//
// Both kernels stream HBM: a thread owns V adjacent channels (one vector
// load) and runs of consecutive tokens. Consecutive lanes own consecutive
// vectors, so a wave reads 1 KiB (forward) or 256 B (backward) of one row per
// load.
//
// Forward: runs of kRun tokens whose row loads (the run's and its W-1 halo
// rows) are all issued before the first is used. A thread loads its taps and
// bias once and takes kFwdPasses runs, one per pass over the tensor, so the
// waves running at any one time cover a narrow band of rows. Measured on
// MI355X, that streams at about the rate of a plain copy; long per-thread
// runs spread the concurrent accesses over ~100 MB and halve it, and loading
// the taps for every short run costs as much again. Halo rows are read again
// by the neighbouring run and mostly hit in L2.
//
// Backward: runs of kBwdRun tokens in the same band-wise passes; a run also
// recomputes the activation gradient of the W - 1 tokens after it, which its
// dx rows need, and its workgroup sums the taps' and bias's gradients over
// its waves.
#include <type_traits>

#include "common.h"

namespace ssmp {

// V adjacent elements of one row moved as a single load or store of
// V * sizeof(T) bytes (V = 1 is the unaligned fallback).
template <int BYTES>
struct RawOf;
template <> struct RawOf<16> { using type = uint4; };
template <> struct RawOf<8> { using type = uint2; };
template <> struct RawOf<4> { using type = uint32_t; };
template <> struct RawOf<2> { using type = uint16_t; };

template <typename T, int V_>
struct Access {
    static constexpr int V = V_;
    using Raw = typename RawOf<V * (int)sizeof(T)>::type;
    struct Arr {
        T v[V];
    };
    static __device__ __forceinline__ Raw load_raw(const T* __restrict__ p) {
        return *reinterpret_cast<const Raw*>(p);
    }
    static __device__ __forceinline__ void unpack(const Raw& r, float (&f)[V]) {
        const Arr a = __builtin_bit_cast(Arr, r);
#pragma unroll
        for (int i = 0; i < V; ++i) f[i] = Elt<T>::ld(a.v, i);
    }
    static __device__ __forceinline__ void load(const T* __restrict__ p, float (&f)[V]) { unpack(load_raw(p), f); }
    static __device__ __forceinline__ void store(T* __restrict__ p, const float (&f)[V]) {
        Arr a;
#pragma unroll
        for (int i = 0; i < V; ++i) Elt<T>::st(a.v, i, f[i]);
        *reinterpret_cast<Raw*>(p) = __builtin_bit_cast(Raw, a);
    }
};

// elements per access: 16 bytes in the forward; 4 in the backward, whose
// per-channel state (taps, window, gradient sums) grows with the vector: at 4
// bytes and 12-token runs a thread holds 89 VGPRs and five waves share a
// SIMD, enough to cover the run's loads (measured at 8-token runs: 0.196 ms
// against 0.225 at 8 bytes, 3 waves, and 0.236 at 2 bytes)
template <typename T> constexpr int kFwdV = 16 / (int)sizeof(T);
template <typename T> constexpr int kBwdV = 4 / (int)sizeof(T);

constexpr int kRun = 8;            // forward: tokens per run
constexpr int kFwdPasses = 4;      // forward: runs per thread, one per pass
// backward: tokens per run. Each run recomputes the activation gradient of
// W - 1 tokens past its end; at 8 tokens that is 3/8 more of that work, at 12
// only 1/4 (measured: 0.176 against 0.197 ms; 10 and 14 tie with 12, 16, 20,
// 24 and 32 are slower as registers grow and fewer waves fit a SIMD)
constexpr int kBwdRun = 12;
constexpr int kConvBwdRuns = 4;    // backward: waves per workgroup, on consecutive runs
constexpr int kConvBwdGroups = 128; // backward: workgroups per 64 vectors (a pass covers 512 runs)

// taps used at token t: k <= kmax (pos[t] caps the look-back at the head)
__device__ __forceinline__ int conv_kmax(int32_t pos_t, int64_t t, int W) {
    int kmax = pos_t;
    if (kmax > W - 1) kmax = W - 1;
    if ((int64_t)kmax > t) kmax = (int)t;
    return kmax;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename T, int V, int W>
__global__ __launch_bounds__(256) void k_conv_fwd(const T* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ b, const int32_t* __restrict__ pos,
                                                  T* __restrict__ u, int64_t T_, int D, int silu) {
    using A = Access<T, V>;
    const int nvec = D / V;
    const int64_t nrun = (T_ + kRun - 1) / kRun;
    const int64_t S = (nrun + kFwdPasses - 1) / kFwdPasses;  // runs per pass
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cv = (int)(gid % nvec);
    const int64_t r0 = gid / nvec;
    if (r0 >= S) return;
    const int d0 = cv * V;

    // wk[k][i]: weight of the tap k tokens back, for channel d0+i
    float wk[4][V], bias[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        bias[i] = b ? b[d0 + i] : 0.0f;
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k][i] = w[(size_t)(d0 + i) * W + (W - 1 - k)];
    }
    // one run; FULL runs (kRun tokens) are straight-line code, so every load
    // stays ahead of the arithmetic
    auto run = [&](auto full_tag, int64_t t0, int nt) {
        constexpr bool FULL = decltype(full_tag)::value;
        // rows t0-3 .. t0+kRun-1; rows outside [0, T) load row t0 and are never selected
        typename A::Raw raw[kRun + 3];
        int32_t pk[kRun];
#pragma unroll
        for (int j = 0; j < kRun + 3; ++j) {
            const int64_t t = t0 - 3 + j;
            const bool in = t >= 0 && (FULL ? j < 3 + kRun : t < T_);
            raw[j] = A::load_raw(x + (size_t)(in ? t : t0) * D + d0);
        }
#pragma unroll
        for (int j = 0; j < kRun; ++j) pk[j] = pos[t0 + ((FULL || j < nt) ? j : 0)];
        // no head within W - 1 tokens before any of the run's tokens: every tap
        // is used, with no per-element selects (heads are rare)
        bool clean = t0 >= W - 1;
#pragma unroll
        for (int j = 0; j < kRun; ++j) clean = clean && pk[j] >= W - 1;
        // window xw[k] = x[t-k]
        float xw[4][V];
#pragma unroll
        for (int k = 1; k < 4; ++k) A::unpack(raw[3 - k], xw[k]);
#pragma unroll
        for (int j = 0; j < kRun; ++j) {
            if (!FULL && j >= nt) break;
            const int64_t t = t0 + j;
            A::unpack(raw[j + 3], xw[0]);
            int kmax = pk[j] < W - 1 ? pk[j] : W - 1;
            if (t0 < W - 1 && kmax > (int)t) kmax = (int)t;  // only the first tokens of the tensor
            float o[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float acc = bias[i];
                if (clean) {
#pragma unroll
                    for (int k = 0; k < W; ++k) acc = __builtin_fmaf(wk[k][i], xw[k][i], acc);
                } else {
#pragma unroll
                    for (int k = 0; k < W; ++k) acc += (k <= kmax) ? wk[k][i] * xw[k][i] : 0.0f;
                }
                o[i] = silu ? acc * sigmoid_fast(acc) : acc;
            }
            A::store(u + (size_t)t * D + d0, o);
#pragma unroll
            for (int k = 3; k > 0; --k)
#pragma unroll
                for (int i = 0; i < V; ++i) xw[k][i] = xw[k - 1][i];
        }
    };
    for (int ps = 0; ps < kFwdPasses; ++ps) {
        const int64_t t0 = (r0 + ps * S) * kRun;
        if (t0 >= T_) break;
        if (t0 + kRun <= T_)
            run(std::true_type{}, t0, kRun);
        else
            run(std::false_type{}, t0, (int)(T_ - t0));
    }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
// For a run [t0, t0 + kRun): gv[t] = du[t] * act'(v[t]) for t in
// [t0, t0 + kRun + W - 1) (the last W - 1 are the next run's, recomputed
// here); dx[s] = sum_k [k <= kmax(s+k)] w_k gv[s+k] for s in the run; dw and
// db collect the run's own tokens. A workgroup is kConvBwdRuns waves on the
// same 64 vectors; wave w takes runs (grp kConvBwdRuns + w) + i G kConvBwdRuns
// for i = 0, 1, ..., so each pass of the G workgroups sweeps a band of
// G kConvBwdRuns consecutive runs. The waves' dw/db sums are added in LDS in
// a fixed order and written to part[grp][j][d] (j = tap k for k < 4, j = 4 for
// the bias).
template <typename T, int V, int W>
__global__ __launch_bounds__(kWave * kConvBwdRuns) void k_conv_bwd(
    const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ b,
    const int32_t* __restrict__ pos, const T* __restrict__ du, T* __restrict__ dx, float* __restrict__ part,
    int64_t T_, int D, int silu) {
    using A = Access<T, V>;
    constexpr int NX = kBwdRun + 2 * (W - 1);  // x rows t0-(W-1) .. t0+kBwdRun+W-2
    constexpr int NG = kBwdRun + W - 1;        // gv of tokens t0 .. t0+kBwdRun+W-2
    __shared__ float red[kConvBwdRuns][5][kWave * V];
    const int nvec = D / V;
    const int nvg = (nvec + kWave - 1) / kWave;  // 64-vector groups
    const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int vg = (int)(blockIdx.x % nvg);
    const int64_t grp = blockIdx.x / nvg;
    const int64_t ngrp = gridDim.x / nvg;
    const int cv = vg * kWave + lane;
    const bool actv = cv < nvec;
    const int d0 = (actv ? cv : 0) * V;
    const int64_t nrun = (T_ + kBwdRun - 1) / kBwdRun;

    float dwp[4][V], dbp[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        dbp[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) dwp[k][i] = 0.0f;
    }
    float wk[4][V], bias[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        bias[i] = b ? b[d0 + i] : 0.0f;
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k][i] = w[(size_t)(d0 + i) * W + (W - 1 - k)];
    }

    // one run; FULL runs (kBwdRun own tokens and all W - 1 tokens after them
    // inside the tensor) are straight-line code, so every load stays ahead of
    // the arithmetic
    auto run = [&](auto full_tag, int64_t t0) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int nt = FULL ? kBwdRun : (int)((T_ - t0 < kBwdRun) ? T_ - t0 : kBwdRun);  // own tokens
        // rows outside [0, T) load row t0 and are never selected
        typename A::Raw rx[NX], rg[NG];
        int32_t pk[NG];
#pragma unroll
        for (int j = 0; j < NX; ++j) {
            const int64_t t = t0 - (W - 1) + j;
            const bool in = t >= 0 && (FULL || t < T_);
            rx[j] = A::load_raw(x + (size_t)(in ? t : t0) * D + d0);
        }
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int64_t t = t0 + j;
            const bool in = FULL || t < T_;
            rg[j] = A::load_raw(du + (size_t)(in ? t : t0) * D + d0);
            pk[j] = pos[in ? t : t0];
        }
        // no head within W - 1 tokens before any token of the run or of its W - 1
        // successors (and all inside the tensor): no per-element selects
        bool clean = FULL && t0 >= W - 1;
#pragma unroll
        for (int j = 0; j < NG; ++j) clean = clean && pk[j] >= W - 1;
        // gv and kmax of tokens t0 .. t0+NG-1 (zero / -1 past the end)
        float gw[NG][V];
        int kw[NG];
        float xw[4][V];
#pragma unroll
        for (int k = 1; k < W; ++k) A::unpack(rx[W - 1 - k], xw[k]);
#pragma unroll
        for (int j = 0; j < NG; ++j) {
            const int64_t t = t0 + j;
            const bool have = FULL || t < T_;
            A::unpack(rx[j + W - 1], xw[0]);
            float g[V];
            A::unpack(rg[j], g);
            int kmax = pk[j] < W - 1 ? pk[j] : W - 1;
            if (t0 < W - 1 && kmax > (int)t) kmax = (int)t;  // only the first tokens of the tensor
            kmax = have ? kmax : -1;
            kw[j] = kmax;
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float v = bias[i];
                if (clean) {
#pragma unroll
                    for (int k = 0; k < W; ++k) v = __builtin_fmaf(wk[k][i], xw[k][i], v);
                } else {
#pragma unroll
                    for (int k = 0; k < W; ++k) v += (k <= kmax) ? wk[k][i] * xw[k][i] : 0.0f;
                }
                float gv = g[i];
                if (silu) {
                    const float sg = sigmoid_fast(v);
                    gv = g[i] * sg * (1.0f + v * (1.0f - sg));
                }
                gv = have ? gv : 0.0f;
                gw[j][i] = gv;
                if (j < kBwdRun && (FULL || j < nt)) {  // dw/db: the run's own tokens
                    if (clean) {
#pragma unroll
                        for (int k = 0; k < W; ++k) dwp[k][i] = __builtin_fmaf(gv, xw[k][i], dwp[k][i]);
                    } else {
#pragma unroll
                        for (int k = 0; k < W; ++k) dwp[k][i] += (k <= kmax) ? gv * xw[k][i] : 0.0f;
                    }
                    dbp[i] += gv;
                }
            }
#pragma unroll
            for (int k = W - 1; k > 0; --k)
#pragma unroll
                for (int i = 0; i < V; ++i) xw[k][i] = xw[k - 1][i];
        }
        // dx[s], s = t0 + j: token s + k feeds tap k when k <= kmax(s + k)
#pragma unroll
        for (int j = 0; j < kBwdRun; ++j) {
            if (!FULL && j >= nt) break;
            float o[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float acc = 0.0f;
                if (clean) {
#pragma unroll
                    for (int k = 0; k < W; ++k) acc = __builtin_fmaf(wk[k][i], gw[j + k][i], acc);
                } else {
#pragma unroll
                    for (int k = 0; k < W; ++k) acc += (k <= kw[j + k]) ? wk[k][i] * gw[j + k][i] : 0.0f;
                }
                o[i] = acc;
            }
            A::store(dx + (size_t)(t0 + j) * D + d0, o);
        }
    };
    // the run index is the same for the whole wave: keep it scalar, so row
    // addresses are a scalar base plus the lane's column offset
    const int64_t rfirst = (int64_t)__builtin_amdgcn_readfirstlane((int)(grp * kConvBwdRuns + wv));
    if (actv) {
        for (int64_t r = rfirst; r < nrun; r += ngrp * kConvBwdRuns) {
            const int64_t t0 = r * kBwdRun;
            if (t0 + kBwdRun + W - 1 <= T_)
                run(std::true_type{}, t0);
            else
                run(std::false_type{}, t0);
        }
    }

    // fixed-order sum of the workgroup's waves
#pragma unroll
    for (int i = 0; i < V; ++i) {
#pragma unroll
        for (int k = 0; k < 4; ++k) red[wv][k][lane * V + i] = dwp[k][i];
        red[wv][4][lane * V + i] = dbp[i];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 5 * kWave * V; e += kWave * kConvBwdRuns) {
        const int j = e / (kWave * V), c = e % (kWave * V);
        const int d = vg * kWave * V + c;
        if (d >= nvec * V) continue;
        float acc = red[0][j][c];
#pragma unroll
        for (int r = 1; r < kConvBwdRuns; ++r) acc += red[r][j][c];
        part[((size_t)grp * 5 + j) * D + d] = acc;
    }
}

// dw[d, W-1-k] = sum_g part[g][k][d];  db[d] = sum_g part[g][4][d]
__global__ __launch_bounds__(256) void k_conv_bwd_reduce(const float* __restrict__ part, int64_t nrun, int D, int W,
                                                         float* __restrict__ dw, float* __restrict__ db) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)5 * D) return;
    const int j = (int)(i / D), d = (int)(i % D);
    if (j < 4 && j >= W) return;
    if (j == 4 && !db) return;
    const float acc = ordered_sum(part + (size_t)j * D + d, nrun, (size_t)5 * D);
    if (j < 4) dw[(size_t)d * W + (W - 1 - j)] = acc;
    else db[d] = acc;
}

// ---------------------------------------------------------------------------
// sequences with a conv context (conv1d_pack_*_states)
// ---------------------------------------------------------------------------
// ctx[s] holds the W-1 inputs before sequence s's first token ((nseq, W-1, D),
// j = 0 the oldest); they stand in for the zeros of the reset. Only the first
// W-1 tokens of a sequence see them, and only its last W-1 inputs make up the
// context it hands on, so the streaming kernels above run unchanged and the
// kernels below, one thread per (sequence, channel), redo the few tokens the
// contexts touch.

// input i of sequence s's extended input [ctx[s]; x[a:e)] (a = cu[s])
template <typename T>
__device__ __forceinline__ float ctx_input(const T* __restrict__ x, const T* __restrict__ ctx, int s, int64_t a,
                                           int64_t i, int D, int W, int d) {
    if (i >= a) return Elt<T>::ld(x, (size_t)i * D + d);
    if (!ctx) return 0.0f;
    return Elt<T>::ld(ctx, ((size_t)s * (W - 1) + (size_t)(i - (a - (W - 1)))) * D + d);
}

// Token range [a, e) of sequence s, clamped into [0, T] with e >= a: with an
// invalid device cu_seqlens (reported by varlen_pack_indices' dev_err) the
// context kernels still only touch rows of the tensors.
__device__ __forceinline__ void seq_range(const int32_t* __restrict__ cu, int s, int64_t T_, int64_t& a, int64_t& e) {
    const int64_t a0 = cu[s], e0 = cu[s + 1];
    a = a0 < 0 ? 0 : (a0 > T_ ? T_ : a0);
    e = e0 < a ? a : (e0 > T_ ? T_ : e0);
}

// forward: outputs of each sequence's first W-1 tokens with the context (ctx
// non-null), and the context each sequence hands on (ctx_out non-null):
// ctx_out[s][j] = input e - (W-1) + j of the extended input (e = cu[s+1])
template <typename T, int W>
__global__ __launch_bounds__(256) void k_conv_fwd_context(const T* __restrict__ x, const float* __restrict__ w,
                                                          const float* __restrict__ b, const int32_t* __restrict__ cu,
                                                          int nseq, const T* __restrict__ ctx, T* __restrict__ u,
                                                          T* __restrict__ ctx_out, int64_t T_, int D, int silu) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)nseq * D) return;
    const int s = (int)(i / D), d = (int)(i % D);
    int64_t a, e;
    seq_range(cu, s, T_, a, e);
    if (ctx) {
        float wk[W];
#pragma unroll
        for (int k = 0; k < W; ++k) wk[k] = w[(size_t)d * W + (W - 1 - k)];
        const float bias = b ? b[d] : 0.0f;
        for (int j = 0; j < W - 1 && a + j < e; ++j) {
            const int64_t t = a + j;
            float acc = bias;
#pragma unroll
            for (int k = 0; k < W; ++k) acc = __builtin_fmaf(wk[k], ctx_input(x, ctx, s, a, t - k, D, W, d), acc);
            Elt<T>::st(u, (size_t)t * D + d, silu ? acc * sigmoid_fast(acc) : acc);
        }
    }
    if (ctx_out) {
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
            Elt<T>::st(ctx_out, ((size_t)s * (W - 1) + j) * D + d, ctx_input(x, ctx, s, a, e - (W - 1) + j, D, W, d));
    }
}

// backward: with a context, the first W-1 tokens' activation gradients change
// (so do dx of those tokens and the tap and bias sums); the handed-on
// context's gradient dctx_out adds to dx of the last W-1 inputs. This kernel
// rewrites dx of those tokens in full, writes the context's gradient dctx,
// and (with a context) per-sequence corrections of the tap and bias sums,
// part[s][j][d] as the streaming kernel's partial rows, which the final
// fixed-order reduction adds after them.
template <typename T, int W>
__global__ __launch_bounds__(256) void k_conv_bwd_context(
    const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ b,
    const int32_t* __restrict__ cu, int nseq, const T* __restrict__ ctx, const T* __restrict__ du,
    const T* __restrict__ dctx_out, T* __restrict__ dx, T* __restrict__ dctx, float* __restrict__ part, int64_t T_,
    int D, int silu) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)nseq * D) return;
    const int s = (int)(i / D), d = (int)(i % D);
    int64_t a, e;
    seq_range(cu, s, T_, a, e);
    float wk[W];
#pragma unroll
    for (int k = 0; k < W; ++k) wk[k] = w[(size_t)d * W + (W - 1 - k)];
    const float bias = b ? b[d] : 0.0f;
    // pre-activation of token t (a <= t < e), with the context or with zeros
    auto pre = [&](int64_t t, const T* c) {
        float acc = bias;
#pragma unroll
        for (int k = 0; k < W; ++k) acc = __builtin_fmaf(wk[k], ctx_input(x, c, s, a, t - k, D, W, d), acc);
        return acc;
    };
    auto grad = [&](int64_t t, float v) {
        const float g = Elt<T>::ld(du, (size_t)t * D + d);
        if (!silu) return g;
        const float sg = sigmoid_fast(v);
        return g * sg * (1.0f + v * (1.0f - sg));
    };
    // gradient of extended input p: taps of the tokens it feeds, plus the
    // handed-on context's gradient if p is among the last W-1 inputs
    auto input_grad = [&](int64_t p) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const int64_t t = p + k;
            if (t >= a && t < e) acc = __builtin_fmaf(wk[k], grad(t, pre(t, ctx)), acc);
        }
        const int64_t jt = p - (e - (W - 1));
        if (dctx_out && jt >= 0 && jt < W - 1) acc += Elt<T>::ld(dctx_out, ((size_t)s * (W - 1) + jt) * D + d);
        return acc;
    };
    const int64_t first_end = ctx ? (a + W - 1 < e ? a + W - 1 : e) : a;
    const int64_t last_start = dctx_out ? (e - (W - 1) > first_end ? e - (W - 1) : first_end) : e;
    for (int64_t p = a; p < first_end; ++p) Elt<T>::st(dx, (size_t)p * D + d, input_grad(p));
    for (int64_t p = last_start; p < e; ++p) Elt<T>::st(dx, (size_t)p * D + d, input_grad(p));
    if (dctx) {
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
            Elt<T>::st(dctx, ((size_t)s * (W - 1) + j) * D + d, input_grad(a - (W - 1) + j));
    }
    if (part) {
        // the streaming kernel summed these tokens with a zero context
        float dwc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, dbc = 0.0f;
        for (int64_t t = a; t < first_end; ++t) {
            const float gr = grad(t, pre(t, ctx));
            const float gz = grad(t, pre(t, nullptr));
            dbc += gr - gz;
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int64_t p = t - k;
                dwc[k] += (p >= a) ? (gr - gz) * Elt<T>::ld(x, (size_t)p * D + d)
                                   : gr * ctx_input(x, ctx, s, a, p, D, W, d);
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) part[((size_t)s * 5 + k) * D + d] = dwc[k];
        part[((size_t)s * 5 + 4) * D + d] = dbc;
    }
}

// workgroups per 64-vector group of the backward (one partial row set each):
// enough for one pass to cover every run of a short input
static int64_t conv_bwd_groups(int64_t T_) {
    const int64_t nrun = (T_ + kBwdRun - 1) / kBwdRun;
    const int64_t need = (nrun + kConvBwdRuns - 1) / kConvBwdRuns;
    return need < kConvBwdGroups ? need : kConvBwdGroups;
}

static bool vec_ok(const void* p, int D, int V, size_t elt) {
    return (D % V == 0) && ((reinterpret_cast<uintptr_t>(p) % (V * elt)) == 0);
}

template <typename T>
static int launch_fwd_context(const void* x, const float* w, const float* b, const int32_t* cu, int nseq,
                              const void* ctx, void* u, void* ctx_out, int64_t T_, int D, int W, int silu,
                              hipStream_t s) {
    const int64_t n = (int64_t)nseq * D;
    const unsigned blocks = (unsigned)((n + 255) / 256);
#define SSMP_CONV_CTX(WX)                                                                                        \
    k_conv_fwd_context<T, WX><<<blocks, 256, 0, s>>>((const T*)x, w, b, cu, nseq, (const T*)ctx, (T*)u,          \
                                                     (T*)ctx_out, T_, D, silu)
    switch (W) {
        case 1: return SSMP_OK;  // no look-back, no context
        case 2: SSMP_CONV_CTX(2); break;
        case 3: SSMP_CONV_CTX(3); break;
        default: SSMP_CONV_CTX(4); break;
    }
#undef SSMP_CONV_CTX
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

template <typename T>
static int launch_bwd_context(const void* x, const float* w, const float* b, const int32_t* cu, int nseq,
                              const void* ctx, const void* du, const void* dctx_out, void* dx, void* dctx,
                              float* part, int64_t T_, int D, int W, int silu, hipStream_t s) {
    const int64_t n = (int64_t)nseq * D;
    const unsigned blocks = (unsigned)((n + 255) / 256);
#define SSMP_CONV_CTX(WX)                                                                                        \
    k_conv_bwd_context<T, WX><<<blocks, 256, 0, s>>>((const T*)x, w, b, cu, nseq, (const T*)ctx, (const T*)du,   \
                                                     (const T*)dctx_out, (T*)dx, (T*)dctx, part, T_, D, silu)
    switch (W) {
        case 1: return SSMP_OK;
        case 2: SSMP_CONV_CTX(2); break;
        case 3: SSMP_CONV_CTX(3); break;
        default: SSMP_CONV_CTX(4); break;
    }
#undef SSMP_CONV_CTX
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

template <typename T>
static int launch_fwd(const void* x, const float* w, const float* b, const int32_t* pos, void* u, int64_t T_, int D,
                      int W, int silu, hipStream_t s) {
    constexpr int VV = kFwdV<T>;
    const bool vec = vec_ok(x, D, VV, sizeof(T)) && vec_ok(u, D, VV, sizeof(T));
    const int V = vec ? VV : 1;
    const int64_t nrun = (T_ + kRun - 1) / kRun;
    const int64_t nthreads = (int64_t)(D / V) * ((nrun + kFwdPasses - 1) / kFwdPasses);
    const int64_t blocks = (nthreads + 255) / 256;
    if (blocks > 0x7fffffff) return SSMP_ERR_SHAPE;
#define SSMP_CONV_FWD(VX, WX) \
    k_conv_fwd<T, VX, WX><<<(unsigned)blocks, 256, 0, s>>>((const T*)x, w, b, pos, (T*)u, T_, D, silu)
#define SSMP_CONV_FWD_W(VX)        \
    switch (W) {                   \
        case 1: SSMP_CONV_FWD(VX, 1); break; \
        case 2: SSMP_CONV_FWD(VX, 2); break; \
        case 3: SSMP_CONV_FWD(VX, 3); break; \
        default: SSMP_CONV_FWD(VX, 4); break; \
    }
    if (vec) {
        SSMP_CONV_FWD_W(VV)
    } else {
        SSMP_CONV_FWD_W(1)
    }
#undef SSMP_CONV_FWD_W
#undef SSMP_CONV_FWD
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

// extra_rows: per-sequence correction rows the context kernel wrote after the
// streaming kernel's partial rows (zero without a context); the context
// kernel runs between the streaming kernel and the reduction.
template <typename T>
static int launch_bwd(const void* x, const float* w, const float* b, const int32_t* pos, const void* du, void* dx,
                      float* dw, float* db, float* part, int64_t T_, int D, int W, int silu, hipStream_t s,
                      int64_t extra_rows = 0, const int32_t* cu = nullptr, int nseq = 0, const void* ctx = nullptr,
                      const void* dctx_out = nullptr, void* dctx = nullptr) {
    constexpr int VV = kBwdV<T>;
    const bool vec = vec_ok(x, D, VV, sizeof(T)) && vec_ok(du, D, VV, sizeof(T)) && vec_ok(dx, D, VV, sizeof(T));
    const int V = vec ? VV : 1;
    const int64_t ngrp = conv_bwd_groups(T_);
    const int64_t nvg = (D / V + kWave - 1) / kWave;
    const int64_t blocks = nvg * ngrp;
    if (blocks > 0x7fffffff) return SSMP_ERR_SHAPE;
#define SSMP_CONV_BWD(VX, WX)                                                  \
    k_conv_bwd<T, VX, WX><<<(unsigned)blocks, kWave * kConvBwdRuns, 0, s>>>( \
        (const T*)x, w, b, pos, (const T*)du, (T*)dx, part, T_, D, silu)
#define SSMP_CONV_BWD_W(VX)                   \
    switch (W) {                              \
        case 1: SSMP_CONV_BWD(VX, 1); break;  \
        case 2: SSMP_CONV_BWD(VX, 2); break;  \
        case 3: SSMP_CONV_BWD(VX, 3); break;  \
        default: SSMP_CONV_BWD(VX, 4); break; \
    }
    if (vec) {
        SSMP_CONV_BWD_W(VV)
    } else {
        SSMP_CONV_BWD_W(1)
    }
#undef SSMP_CONV_BWD_W
#undef SSMP_CONV_BWD
    SSMP_LAUNCH_CHECK();
    if (cu) {
        const int st = launch_bwd_context<T>(x, w, b, cu, nseq, ctx, du, dctx_out, dx, dctx,
                                             extra_rows ? part + (size_t)ngrp * 5 * D : nullptr, T_, D, W, silu, s);
        if (st) return st;
    }
    k_conv_bwd_reduce<<<(unsigned)((5 * (int64_t)D + 255) / 256), 256, 0, s>>>(part, ngrp + extra_rows, D, W, dw,
                                                                               db);
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

static int check_conv_args(int64_t T_, int D, int W, int dtype) {
    if (T_ < 0 || D < 1) return SSMP_ERR_SHAPE;
    if (T_ > 0 && (T_ * (int64_t)D) >= (int64_t(1) << 40)) return SSMP_ERR_SHAPE;
    if (W < 1 || W > 4) return SSMP_ERR_UNSUPPORTED;
    if (dtype != SSMP_F32 && dtype != SSMP_BF16) return SSMP_ERR_UNSUPPORTED;
    return SSMP_OK;
}

}  // namespace ssmp

extern "C" int conv1d_pack_fwd(const void* x, const float* w, const float* b, const int32_t* pos, void* u,
                               int64_t T, int32_t D, int32_t W, int32_t dtype, int32_t silu, void* stream) {
    using namespace ssmp;
    int st = check_conv_args(T, D, W, dtype);
    if (st) return st;
    if (T == 0) return SSMP_OK;
    if (!x || !w || !pos || !u) return SSMP_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return dtype == SSMP_BF16 ? launch_fwd<uint16_t>(x, w, b, pos, u, T, D, W, silu != 0, s)
                              : launch_fwd<float>(x, w, b, pos, u, T, D, W, silu != 0, s);
}

extern "C" int conv1d_pack_fwd_states(const void* x, const float* w, const float* b, const int32_t* pos, void* u,
                                      int64_t T, int32_t D, int32_t W, int32_t dtype, int32_t silu,
                                      const int32_t* cu_seqlens, int32_t nseq, const void* conv_initial,
                                      void* conv_final, void* stream) {
    using namespace ssmp;
    int st = check_conv_args(T, D, W, dtype);
    if (st) return st;
    const bool states = conv_initial || conv_final;
    if (states) {
        if (!cu_seqlens) return SSMP_ERR_NULL;
        if (nseq < 1 || (int64_t)nseq * D >= (int64_t(1) << 40)) return SSMP_ERR_SHAPE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T > 0) {
        if (!x || !w || !pos || !u) return SSMP_ERR_NULL;
        st = dtype == SSMP_BF16 ? launch_fwd<uint16_t>(x, w, b, pos, u, T, D, W, silu != 0, s)
                                : launch_fwd<float>(x, w, b, pos, u, T, D, W, silu != 0, s);
        if (st) return st;
    } else if (!w) {
        return SSMP_ERR_NULL;
    }
    if (!states) return SSMP_OK;
    return dtype == SSMP_BF16 ? launch_fwd_context<uint16_t>(x, w, b, cu_seqlens, nseq, conv_initial, u, conv_final,
                                                             T, D, W, silu != 0, s)
                              : launch_fwd_context<float>(x, w, b, cu_seqlens, nseq, conv_initial, u, conv_final, T,
                                                          D, W, silu != 0, s);
}

extern "C" size_t conv1d_pack_bwd_workspace_bytes(int64_t T, int32_t D, int32_t W) {
    (void)W;
    if (T <= 0 || D <= 0) return 0;
    return (size_t)ssmp::conv_bwd_groups(T) * 5 * (size_t)D * sizeof(float);
}

extern "C" int conv1d_pack_bwd(const void* x, const float* w, const float* b, const int32_t* pos, const void* du,
                               void* dx, float* dw, float* db, void* workspace, size_t workspace_bytes, int64_t T,
                               int32_t D, int32_t W, int32_t dtype, int32_t silu, void* stream) {
    using namespace ssmp;
    int st = check_conv_args(T, D, W, dtype);
    if (st) return st;
    if (!w || !dw) return SSMP_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        // empty input: the sums are zero
        if ((st = zero_f32(dw, (int64_t)D * W, s))) return st;
        return zero_f32(db, D, s);
    }
    if (!x || !pos || !du || !dx) return SSMP_ERR_NULL;
    if (!workspace || workspace_bytes < conv1d_pack_bwd_workspace_bytes(T, D, W)) return SSMP_ERR_WORKSPACE;
    return dtype == SSMP_BF16
               ? launch_bwd<uint16_t>(x, w, b, pos, du, dx, dw, db, (float*)workspace, T, D, W, silu != 0, s)
               : launch_bwd<float>(x, w, b, pos, du, dx, dw, db, (float*)workspace, T, D, W, silu != 0, s);
}

extern "C" size_t conv1d_pack_bwd_states_workspace_bytes(int64_t T, int32_t D, int32_t W, int32_t nseq) {
    if (T <= 0 || D <= 0 || nseq < 0) return 0;
    return conv1d_pack_bwd_workspace_bytes(T, D, W) + (size_t)nseq * 5 * (size_t)D * sizeof(float);
}

extern "C" int conv1d_pack_bwd_states(const void* x, const float* w, const float* b, const int32_t* pos,
                                      const void* du, void* dx, float* dw, float* db, void* workspace,
                                      size_t workspace_bytes, int64_t T, int32_t D, int32_t W, int32_t dtype,
                                      int32_t silu, const int32_t* cu_seqlens, int32_t nseq,
                                      const void* conv_initial, const void* dconv_final, void* dconv_initial,
                                      void* stream) {
    using namespace ssmp;
    const bool states = conv_initial || dconv_final || dconv_initial;
    if (!states)
        return conv1d_pack_bwd(x, w, b, pos, du, dx, dw, db, workspace, workspace_bytes, T, D, W, dtype, silu,
                               stream);
    int st = check_conv_args(T, D, W, dtype);
    if (st) return st;
    if (!w || !dw || !cu_seqlens) return SSMP_ERR_NULL;
    if (nseq < 1 || (int64_t)nseq * D >= (int64_t(1) << 40)) return SSMP_ERR_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        // no tokens: the sums are zero; every sequence hands the gradient of
        // its handed-on context back to its own context
        if ((st = zero_f32(dw, (int64_t)D * W, s))) return st;
        if ((st = zero_f32(db, D, s))) return st;
        if (!dconv_initial) return SSMP_OK;
        return dtype == SSMP_BF16
                   ? launch_bwd_context<uint16_t>(x, w, b, cu_seqlens, nseq, conv_initial, du, dconv_final, dx,
                                                  dconv_initial, nullptr, T, D, W, silu != 0, s)
                   : launch_bwd_context<float>(x, w, b, cu_seqlens, nseq, conv_initial, du, dconv_final, dx,
                                               dconv_initial, nullptr, T, D, W, silu != 0, s);
    }
    if (!x || !pos || !du || !dx) return SSMP_ERR_NULL;
    if (!workspace || workspace_bytes < conv1d_pack_bwd_states_workspace_bytes(T, D, W, nseq))
        return SSMP_ERR_WORKSPACE;
    const int64_t extra = (conv_initial && W > 1) ? nseq : 0;
    return dtype == SSMP_BF16
               ? launch_bwd<uint16_t>(x, w, b, pos, du, dx, dw, db, (float*)workspace, T, D, W, silu != 0, s, extra,
                                      cu_seqlens, nseq, conv_initial, dconv_final, dconv_initial)
               : launch_bwd<float>(x, w, b, pos, du, dx, dw, db, (float*)workspace, T, D, W, silu != 0, s, extra,
                                   cu_seqlens, nseq, conv_initial, dconv_final, dconv_initial);
}
