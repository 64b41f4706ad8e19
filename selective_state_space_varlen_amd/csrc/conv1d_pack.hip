// conv1d_pack forward and backward: causal depthwise conv of width W <= 4 that
// stops at each sequence's head token.
//
// Shanghai AI Lab article on packed variable-length Mamba-1 training
// (gitcode.csdn.net/69d8cc1b54b52172bc6872cb.html), section "conv1d_pack 算子":
// the conv looks back W-1 tokens and terminates early at a head; the backward
// stops dx and dweight the same way, taking the reverse position from the
// position index W-1 tokens ahead.
//
// Both kernels stream HBM: a thread owns V adjacent channels (one 16-byte
// vector) and a run of RT consecutive tokens, slides a W-token window of x in
// registers, and reads the per-token position once per token (the same
// address for the whole wave). Consecutive lanes own consecutive vectors, so
// a wave reads 1 KiB of one row per load. Tokens are taken in batches of kG
// whose loads are all issued before the first is used, so each wave keeps
// kG (forward) or 2 kG (backward) row loads in flight.
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

// elements per access: 16 bytes in the forward; 8 in the backward, whose
// per-channel state (taps, window, gradient sums) would otherwise cost two
// waves per SIMD
template <typename T> constexpr int kFwdV = 16 / (int)sizeof(T);
template <typename T> constexpr int kBwdV = 8 / (int)sizeof(T);

constexpr int kConvFwdRun = 32;   // tokens per thread, forward
constexpr int kConvBwdRun = 64;   // tokens per thread, backward
constexpr int kConvBwdRuns = 4;   // runs per backward workgroup (summed there before the partials)
constexpr int kG = 8;             // tokens per load batch
static_assert(kConvFwdRun % kG == 0 && kConvBwdRun % kG == 0, "runs hold whole batches");

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
template <typename T, int V>
__global__ __launch_bounds__(256) void k_conv_fwd(const T* __restrict__ x, const float* __restrict__ w,
                                                  const float* __restrict__ b, const int32_t* __restrict__ pos,
                                                  T* __restrict__ u, int64_t T_, int D, int W, int silu) {
    using A = Access<T, V>;
    const int nvec = D / V;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cv = (int)(gid % nvec);
    const int64_t t0 = (gid / nvec) * kConvFwdRun;
    if (t0 >= T_) return;
    const int64_t t1 = (t0 + kConvFwdRun < T_) ? t0 + kConvFwdRun : T_;
    const int d0 = cv * V;

    // wk[k][i]: weight of the tap k tokens back, for channel d0+i (0 beyond W)
    float wk[4][V], bias[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        bias[i] = b ? b[d0 + i] : 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) wk[k][i] = (k < W) ? w[(size_t)(d0 + i) * W + (W - 1 - k)] : 0.0f;
    }
    // window xw[k] = x[t-k]; tokens before 0 are never selected
    float xw[4][V];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        const int64_t tk = t0 - k;
        if (tk >= 0) {
            A::load(x + (size_t)tk * D + d0, xw[k]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) xw[k][i] = 0.0f;
        }
    }
    for (int64_t tb = t0; tb < t1; tb += kG) {
        const int ng = (int)((t1 - tb < kG) ? t1 - tb : kG);
        typename A::Raw raw[kG];
        int32_t pk[kG];
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            const int64_t t = tb + (g < ng ? g : ng - 1);  // a short batch repeats its last token
            raw[g] = A::load_raw(x + (size_t)t * D + d0);
            pk[g] = pos[t];
        }
#pragma unroll
        for (int g = 0; g < kG; ++g) {
            if (g >= ng) break;
            const int64_t t = tb + g;
            A::unpack(raw[g], xw[0]);
            const int kmax = conv_kmax(pk[g], t, W);
            float o[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float acc = bias[i];
#pragma unroll
                for (int k = 0; k < 4; ++k) acc += (k <= kmax) ? wk[k][i] * xw[k][i] : 0.0f;
                o[i] = silu ? acc * sigmoid_fast(acc) : acc;
            }
            A::store(u + (size_t)t * D + d0, o);
#pragma unroll
            for (int k = 3; k > 0; --k)
#pragma unroll
                for (int i = 0; i < V; ++i) xw[k][i] = xw[k - 1][i];
        }
    }
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------
// Per thread: tokens [t0, t1). gv[t] = du[t] * act'(v[t]) is produced for
// t in [t0, min(t1 + 3, T)); dx[s] for s in [t0, t1) collects
// sum_k [k <= kmax(s+k)] w_k gv[s+k], emitted once gv[s+3] is known (the
// last four gv and their kmax are kept). dw and db sums over [t0, t1) are
// added over the workgroup's kConvBwdRuns runs in LDS, in a fixed order, and
// written to part[group][j][d] (j = tap k for k < 4, j = 4 for the bias).
// A workgroup is kConvBwdRuns waves: the same 64 vectors, consecutive runs.
template <typename T, int V>
__global__ __launch_bounds__(kWave * kConvBwdRuns) void k_conv_bwd(
    const T* __restrict__ x, const float* __restrict__ w, const float* __restrict__ b,
    const int32_t* __restrict__ pos, const T* __restrict__ du, T* __restrict__ dx, float* __restrict__ part,
    int64_t T_, int D, int W, int silu) {
    using A = Access<T, V>;
    __shared__ float red[kConvBwdRuns][5][kWave * V];
    const int nvec = D / V;
    const int nvg = (nvec + kWave - 1) / kWave;  // 64-vector groups
    const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int vg = (int)(blockIdx.x % nvg);
    const int64_t grp = blockIdx.x / nvg;           // workgroup's run group
    const int cv = vg * kWave + lane;
    const bool actv = cv < nvec;
    const int64_t run = grp * kConvBwdRuns + wv;
    const int64_t t0 = run * kConvBwdRun;
    const int64_t t1 = (t0 + kConvBwdRun < T_) ? t0 + kConvBwdRun : T_;
    const int64_t tend = (t1 + 3 < T_) ? t1 + 3 : T_;
    const int d0 = (actv ? cv : 0) * V;

    float dwp[4][V], dbp[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        dbp[i] = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) dwp[k][i] = 0.0f;
    }
    if (actv && t0 < T_) {
        float wk[4][V], bias[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            bias[i] = b ? b[d0 + i] : 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) wk[k][i] = (k < W) ? w[(size_t)(d0 + i) * W + (W - 1 - k)] : 0.0f;
        }
        float xw[4][V];
#pragma unroll
        for (int k = 1; k < 4; ++k) {
            const int64_t tk = t0 - k;
            if (tk >= 0) {
                A::load(x + (size_t)tk * D + d0, xw[k]);
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) xw[k][i] = 0.0f;
            }
        }
        // gw[j] = gv[t-j], kw[j] = kmax(t-j) for the last four tokens (gv = 0 before t0)
        float gw[4][V];
        int kw[4] = {-1, -1, -1, -1};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < V; ++i) gw[j][i] = 0.0f;

        // one token step: shift the windows in, gv of token t (zero past tend), dx[t-3]
        auto step = [&](int64_t t, bool have, const float (&g)[V], int kmax) {
#pragma unroll
            for (int j = 3; j > 0; --j) {
                kw[j] = kw[j - 1];
#pragma unroll
                for (int i = 0; i < V; ++i) gw[j][i] = gw[j - 1][i];
            }
            kw[0] = have ? kmax : -1;
            const bool own = t < t1;  // dw/db sums only over this thread's tokens
#pragma unroll
            for (int i = 0; i < V; ++i) {
                float gv = 0.0f;
                if (have) {
                    float v = bias[i];
#pragma unroll
                    for (int k = 0; k < 4; ++k) v += (k <= kmax) ? wk[k][i] * xw[k][i] : 0.0f;
                    gv = g[i];
                    if (silu) {
                        const float sg = sigmoid_fast(v);
                        gv = g[i] * sg * (1.0f + v * (1.0f - sg));
                    }
                    if (own) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) dwp[k][i] += (k <= kmax) ? gv * xw[k][i] : 0.0f;
                        dbp[i] += gv;
                    }
                }
                gw[0][i] = gv;
            }
            if (have) {
#pragma unroll
                for (int k = 3; k > 0; --k)
#pragma unroll
                    for (int i = 0; i < V; ++i) xw[k][i] = xw[k - 1][i];
            }
            // dx[s], s = t - 3: token s + k feeds tap k when k <= kmax(s + k)
            const int64_t s = t - 3;
            if (s >= t0 && s < t1) {
                float o[V];
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    float acc = 0.0f;
#pragma unroll
                    for (int k = 0; k < 4; ++k) acc += (k <= kw[3 - k]) ? wk[k][i] * gw[3 - k][i] : 0.0f;
                    o[i] = acc;
                }
                A::store(dx + (size_t)s * D + d0, o);
            }
        };

        for (int64_t tb = t0; tb < tend; tb += kG) {
            const int ng = (int)((tend - tb < kG) ? tend - tb : kG);
            typename A::Raw rx[kG], rg[kG];
            int32_t pk[kG];
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                const int64_t t = tb + (g < ng ? g : ng - 1);  // a short batch repeats its last token
                rx[g] = A::load_raw(x + (size_t)t * D + d0);
                rg[g] = A::load_raw(du + (size_t)t * D + d0);
                pk[g] = pos[t];
            }
#pragma unroll
            for (int g = 0; g < kG; ++g) {
                if (g >= ng) break;
                const int64_t t = tb + g;
                float gg[V];
                A::unpack(rx[g], xw[0]);
                A::unpack(rg[g], gg);
                step(t, true, gg, conv_kmax(pk[g], t, W));
            }
        }
        // the tensor ends before t1 + 3: flush the last dx rows
        const float zero[V] = {};
        for (int64_t t = tend; t < t1 + 3; ++t) step(t, false, zero, -1);
    }

    // fixed-order sum of the workgroup's runs
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

// run groups of the backward (one partial row set each)
static int64_t conv_bwd_groups(int64_t T_) {
    const int64_t span = (int64_t)kConvBwdRun * kConvBwdRuns;
    return (T_ + span - 1) / span;
}

static bool vec_ok(const void* p, int D, int V, size_t elt) {
    return (D % V == 0) && ((reinterpret_cast<uintptr_t>(p) % (V * elt)) == 0);
}

template <typename T>
static int launch_fwd(const void* x, const float* w, const float* b, const int32_t* pos, void* u, int64_t T_, int D,
                      int W, int silu, hipStream_t s) {
    constexpr int VV = kFwdV<T>;
    const bool vec = vec_ok(x, D, VV, sizeof(T)) && vec_ok(u, D, VV, sizeof(T));
    const int V = vec ? VV : 1;
    const int64_t nthreads = (int64_t)(D / V) * ((T_ + kConvFwdRun - 1) / kConvFwdRun);
    const int64_t blocks = (nthreads + 255) / 256;
    if (blocks > 0x7fffffff) return SSMP_ERR_SHAPE;
    if (vec)
        k_conv_fwd<T, VV><<<(unsigned)blocks, 256, 0, s>>>((const T*)x, w, b, pos, (T*)u, T_, D, W, silu);
    else
        k_conv_fwd<T, 1><<<(unsigned)blocks, 256, 0, s>>>((const T*)x, w, b, pos, (T*)u, T_, D, W, silu);
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

template <typename T>
static int launch_bwd(const void* x, const float* w, const float* b, const int32_t* pos, const void* du, void* dx,
                      float* dw, float* db, float* part, int64_t T_, int D, int W, int silu, hipStream_t s) {
    constexpr int VV = kBwdV<T>;
    const bool vec = vec_ok(x, D, VV, sizeof(T)) && vec_ok(du, D, VV, sizeof(T)) && vec_ok(dx, D, VV, sizeof(T));
    const int V = vec ? VV : 1;
    const int64_t ngrp = conv_bwd_groups(T_);
    const int64_t nvg = (D / V + kWave - 1) / kWave;
    const int64_t blocks = nvg * ngrp;
    if (blocks > 0x7fffffff) return SSMP_ERR_SHAPE;
    if (vec)
        k_conv_bwd<T, VV><<<(unsigned)blocks, kWave * kConvBwdRuns, 0, s>>>(
            (const T*)x, w, b, pos, (const T*)du, (T*)dx, part, T_, D, W, silu);
    else
        k_conv_bwd<T, 1><<<(unsigned)blocks, kWave * kConvBwdRuns, 0, s>>>(
            (const T*)x, w, b, pos, (const T*)du, (T*)dx, part, T_, D, W, silu);
    SSMP_LAUNCH_CHECK();
    k_conv_bwd_reduce<<<(unsigned)((5 * (int64_t)D + 255) / 256), 256, 0, s>>>(part, ngrp, D, W, dw, db);
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
        if (hipMemsetAsync(dw, 0, sizeof(float) * (size_t)D * W, s) != hipSuccess) return SSMP_ERR_HIP;
        if (db && hipMemsetAsync(db, 0, sizeof(float) * (size_t)D, s) != hipSuccess) return SSMP_ERR_HIP;
        return SSMP_OK;
    }
    if (!x || !pos || !du || !dx) return SSMP_ERR_NULL;
    if (!workspace || workspace_bytes < conv1d_pack_bwd_workspace_bytes(T, D, W)) return SSMP_ERR_WORKSPACE;
    return dtype == SSMP_BF16
               ? launch_bwd<uint16_t>(x, w, b, pos, du, dx, dw, db, (float*)workspace, T, D, W, silu != 0, s)
               : launch_bwd<float>(x, w, b, pos, du, dx, dw, db, (float*)workspace, T, D, W, silu != 0, s);
}
