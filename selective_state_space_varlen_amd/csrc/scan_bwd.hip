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
//   ddelta_t = u_t sum_n dh_t B_t[n] + sum_n [not head] A dh_t a_t h_{t-1}
//   dA    += [not head] delta_t dh_t a_t h_{t-1}       dDskip += g_t u_t
//   dz_t   = dout_t y_t s (1 + z_t (1 - s)),  s = sigmoid(z_t)
//
// Time parallelism mirrors the forward, in reverse: a chunk's carry out of
// its first token is c_out = P' c_in + S' with
//   S' = sum_{s < first head} (prod_{r=t0..s} a_r) g_s C_s,  P' = prod a (0 if a head)
// which one forward sweep over the chunk's leading tokens yields. A
// sequential pass over chunks (right to left) turns these into the carry
// entering each chunk. The main kernel then walks each chunk backwards in
// kCK-token blocks: it restarts from the forward's checkpoint, rebuilds the
// states at kK-token sub-chunk starts (kept in LDS), and for each sub-chunk
// replays kK tokens with their states and decays held in VGPRs before
// running the reverse step over them. dB and dC (sums over channels) are
// reduced across the wave through LDS and written per channel group; dA and
// dDskip are written per chunk; small kernels finish both sums in a fixed
// order, so results are deterministic.
#include "scan_common.h"

namespace ssmp {

// ---------------------------------------------------------------------------
// 1. reverse-carry summaries
// ---------------------------------------------------------------------------
template <typename T, int NS>
__global__ __launch_bounds__(64) void k_scan_bwd_summary(const T* __restrict__ delta, const float* __restrict__ A,
                                                         const T* __restrict__ C, const T* __restrict__ z,
                                                         const T* __restrict__ dout, const int32_t* __restrict__ pos,
                                                         float* __restrict__ Pr, float* __restrict__ Sr, int64_t T_,
                                                         int D) {
    const int lane = threadIdx.x;
    const Tile tl = tile_of(D);
    const int d = tl.g * kWave + lane;
    const bool act = d < D;
    const int dd = act ? d : D - 1;
    const int64_t c = tl.c;
    const int64_t t0 = c * kLC;
    const int64_t t1 = (t0 + kLC < T_) ? t0 + kLC : T_;
    if (c == 0) return;            // nothing to the left
    if (pos[t0] == 0) return;      // starts at a head: carries nothing out

    // first head in (t0, t1)
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
    const bool gate = z != nullptr;
    float A2[NS], pf[NS], sr[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        A2[n] = A[(size_t)dd * NS + n] * kLog2e;
        pf[n] = 1.0f;
        sr[n] = 0.0f;
    }
    for (int64_t t = t0; t < fh; ++t) {
        const size_t e = (size_t)t * D + dd;
        const float dt = Elt<T>::ld(delta, e);
        float g = Elt<T>::ld(dout, e);
        if (gate) {
            const float zz = Elt<T>::ld(z, e);
            g *= zz * sigmoid_fast(zz);
        }
        float Cv[NS];
        load_row<NS>(C + (size_t)t * NS, Cv);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            pf[n] *= exp2_fast(dt * A2[n]);
            sr[n] = __builtin_fmaf(pf[n], g * Cv[n], sr[n]);
        }
    }
    if (act) {
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const size_t o = ((size_t)c * NS + n) * D + d;
            Pr[o] = (fh < t1) ? 0.0f : pf[n];
            Sr[o] = sr[n];
        }
    }
}

// ---------------------------------------------------------------------------
// 2. carries, right to left: cin[c] = carry entering chunk c from chunk c+1
// ---------------------------------------------------------------------------
template <int NS>
__global__ __launch_bounds__(256) void k_scan_bwd_carry(const float* __restrict__ Pr, const float* __restrict__ Sr,
                                                        const int32_t* __restrict__ pos, float* __restrict__ cin,
                                                        int D, int64_t nchunk) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t ND = (int64_t)NS * D;
    if (i >= ND) return;
    float cc = 0.0f;
    for (int64_t c = nchunk - 1; c >= 0; --c) {
        cin[(size_t)c * ND + i] = cc;
        if (c == 0) break;
        if (pos[c * kLC] == 0) {
            cc = 0.0f;
        } else {
            const float Pc = Pr[(size_t)c * ND + i], Sc = Sr[(size_t)c * ND + i];
            cc = (Pc == 0.0f) ? Sc : __builtin_fmaf(Pc, cc, Sc);  // select at heads, as in the forward
        }
    }
}

// ---------------------------------------------------------------------------
// 3. the reverse pass
// ---------------------------------------------------------------------------
template <typename T, int NS>
struct BwdArgs {
    const T* u;
    const T* delta;
    const float* A;
    const T* B;
    const T* C;
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
    float* dBC;
    int64_t T_;
    int D;
};

// Forward step of one token (shared by the replays).
template <typename T, int NS>
__device__ __forceinline__ void fwd_step(const BwdArgs<T, NS>& p, int64_t t, int dd, const float (&A2)[NS],
                                         float (&h)[NS]) {
    const size_t e = (size_t)t * p.D + dd;
    const float dt = Elt<T>::ld(p.delta, e);
    const float dtu = dt * Elt<T>::ld(p.u, e);
    float Bv[NS];
    load_row<NS>(p.B + (size_t)t * NS, Bv);
    if (p.pos[t] == 0) {
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = 0.0f;
    }
#pragma unroll
    for (int n = 0; n < NS; ++n) h[n] = __builtin_fmaf(exp2_fast(dt * A2[n]), h[n], dtu * Bv[n]);
}

constexpr int kRedStride = kWave + 4;  // LDS row stride (floats) of the dB/dC transpose

template <typename T, int NS>
__global__ __launch_bounds__(64) void k_scan_bwd_main(BwdArgs<T, NS> p) {
    constexpr int NSUB = kCK / kK;
    __shared__ float sub[NSUB > 1 ? NSUB - 1 : 1][NS][kWave];
    __shared__ __attribute__((aligned(16))) float red[2 * NS][kRedStride];

    const int lane = threadIdx.x;
    const Tile tl = tile_of(p.D);
    const int g = tl.g;
    const int d = g * kWave + lane;
    const bool act = d < p.D;
    const int dd = act ? d : p.D - 1;
    const int64_t c = tl.c;
    const int64_t t0 = c * kLC;
    const int64_t t1 = (t0 + kLC < p.T_) ? t0 + kLC : p.T_;
    const size_t ND = (size_t)NS * p.D;
    const bool gate = p.z != nullptr;

    float A2[NS], carry[NS], dA[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        A2[n] = p.A[(size_t)dd * NS + n] * kLog2e;
        carry[n] = p.cin[(size_t)c * ND + (size_t)n * p.D + dd];
        dA[n] = 0.0f;
    }
    const float Dv = p.Dskip ? p.Dskip[dd] : 0.0f;
    float dDacc = 0.0f;

    const int64_t nblk = (t1 - t0 + kCK - 1) / kCK;
    for (int64_t jb = nblk - 1; jb >= 0; --jb) {
        const int64_t tb0 = t0 + jb * kCK;
        const int64_t tb1 = (tb0 + kCK < t1) ? tb0 + kCK : t1;
        const int nsub = (int)((tb1 - tb0 + kK - 1) / kK);
        const float* hb = p.ckpt + (size_t)(tb0 / kCK) * ND;

        // states entering sub-chunks 1..nsub-1
        if (nsub > 1) {
            float h[NS];
#pragma unroll
            for (int n = 0; n < NS; ++n) h[n] = hb[(size_t)n * p.D + dd];
            for (int i = 1; i < nsub; ++i) {
#pragma unroll
                for (int k = 0; k < kK; ++k) fwd_step<T, NS>(p, tb0 + (int64_t)(i - 1) * kK + k, dd, A2, h);
#pragma unroll
                for (int n = 0; n < NS; ++n) sub[i - 1][n][lane] = h[n];
            }
        }

        for (int i = nsub - 1; i >= 0; --i) {
            const int64_t ts0 = tb0 + (int64_t)i * kK;
            const int ns = (int)((ts0 + kK < tb1) ? kK : tb1 - ts0);
            float hp0[NS];
            if (i == 0) {
#pragma unroll
                for (int n = 0; n < NS; ++n) hp0[n] = hb[(size_t)n * p.D + dd];
            } else {
#pragma unroll
                for (int n = 0; n < NS; ++n) hp0[n] = sub[i - 1][n][lane];
            }
            // replay: states hh[k] and decays aa[k] of the sub-chunk's tokens
            float hh[kK][NS], aa[kK][NS], yk[kK];
            {
                float h[NS];
#pragma unroll
                for (int n = 0; n < NS; ++n) h[n] = hp0[n];
#pragma unroll
                for (int k = 0; k < kK; ++k) {
                    if (k < ns) {
                        const int64_t t = ts0 + k;
                        const size_t e = (size_t)t * p.D + dd;
                        const float dt = Elt<T>::ld(p.delta, e);
                        const float uu = Elt<T>::ld(p.u, e);
                        const float dtu = dt * uu;
                        float Bv[NS], Cv[NS];
                        load_row<NS>(p.B + (size_t)t * NS, Bv);
                        load_row<NS>(p.C + (size_t)t * NS, Cv);
                        if (p.pos[t] == 0) {
#pragma unroll
                            for (int n = 0; n < NS; ++n) h[n] = 0.0f;
                        }
                        float y = 0.0f;
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            const float a = exp2_fast(dt * A2[n]);
                            aa[k][n] = a;
                            h[n] = __builtin_fmaf(a, h[n], dtu * Bv[n]);
                            hh[k][n] = h[n];
                            y = __builtin_fmaf(Cv[n], h[n], y);
                        }
                        yk[k] = __builtin_fmaf(Dv, uu, y);
                    }
                }
            }
            // reverse over the sub-chunk
#pragma unroll
            for (int k = kK - 1; k >= 0; --k) {
                if (k < ns) {
                    const int64_t t = ts0 + k;
                    const size_t e = (size_t)t * p.D + dd;
                    const float dt = Elt<T>::ld(p.delta, e);
                    const float uu = Elt<T>::ld(p.u, e);
                    const float dtu = dt * uu;
                    const float go = Elt<T>::ld(p.dout, e);
                    float gg = go, dzv = 0.0f;
                    if (gate) {
                        const float zz = Elt<T>::ld(p.z, e);
                        const float sg = sigmoid_fast(zz);
                        gg = go * zz * sg;
                        dzv = go * yk[k] * sg * (1.0f + zz * (1.0f - sg));
                    }
                    float Bv[NS], Cv[NS];
                    load_row<NS>(p.B + (size_t)t * NS, Bv);
                    load_row<NS>(p.C + (size_t)t * NS, Cv);
                    const bool head = p.pos[t] == 0;
                    float sumB = 0.0f, sumAr = 0.0f;
                    const float gm = act ? gg : 0.0f;  // inactive lanes add nothing to dB/dC
                    if (head) {
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            const float dh = __builtin_fmaf(gg, Cv[n], carry[n]);
                            red[n][lane] = act ? dh * dtu : 0.0f;   // dB row
                            red[NS + n][lane] = gm * hh[k][n];        // dC row
                            sumB = __builtin_fmaf(dh, Bv[n], sumB);
                            carry[n] = 0.0f;
                        }
                    } else {
#pragma unroll
                        for (int n = 0; n < NS; ++n) {
                            const float dh = __builtin_fmaf(gg, Cv[n], carry[n]);
                            red[n][lane] = act ? dh * dtu : 0.0f;   // dB row
                            red[NS + n][lane] = gm * hh[k][n];        // dC row
                            sumB = __builtin_fmaf(dh, Bv[n], sumB);
                            const float cc = aa[k][n] * dh;
                            const float hprev = (k == 0) ? hp0[n] : hh[k > 0 ? k - 1 : 0][n];
                            const float r = cc * hprev;
                            sumAr = __builtin_fmaf(r, A2[n], sumAr);
                            dA[n] = __builtin_fmaf(r, dt, dA[n]);
                            carry[n] = cc;
                        }
                    }
                    const float duv = __builtin_fmaf(gg, Dv, dt * sumB);
                    const float ddv = __builtin_fmaf(uu, sumB, sumAr * kLn2);
                    dDacc = __builtin_fmaf(gg, uu, dDacc);
                    if (act) {
                        Elt<T>::st(p.du, (size_t)t * p.D + d, duv);
                        Elt<T>::st(p.ddelta, (size_t)t * p.D + d, ddv);
                        if (gate) Elt<T>::st(p.dz, (size_t)t * p.D + d, dzv);
                    }
                    // dB/dC: sum the wave's 64 channels. Lane l adds half a row
                    // (value l/2, channels 32*(l%2) ..) and its neighbour the other.
                    __syncthreads();
                    const int j = lane >> 1, hf = lane & 1;
                    float v = 0.0f;
                    if (j < 2 * NS) {
                        const float4* row = reinterpret_cast<const float4*>(&red[j][hf * 32]);
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const float4 r4 = row[q];
                            v += (r4.x + r4.y) + (r4.z + r4.w);
                        }
                    }
                    v += __shfl_xor(v, 1);
                    if (hf == 0 && j < 2 * NS) p.dBC[((size_t)g * p.T_ + t) * (2 * NS) + j] = v;
                    __syncthreads();
                }
            }
        }
    }
    if (act) {
#pragma unroll
        for (int n = 0; n < NS; ++n) p.dApart[(size_t)c * ND + (size_t)n * p.D + d] = dA[n];
        p.dDpart[(size_t)c * p.D + d] = dDacc;
    }
}

// ---------------------------------------------------------------------------
// 4. fixed-order sums
// ---------------------------------------------------------------------------
template <int NS>
__global__ __launch_bounds__(256) void k_scan_bwd_reduce_params(const float* __restrict__ dApart,
                                                                const float* __restrict__ dDpart, int64_t nchunk,
                                                                int D, float* __restrict__ dA,
                                                                float* __restrict__ dD) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // n*D + d
    const int64_t ND = (int64_t)NS * D;
    if (i < ND) {
        float acc = 0.0f;
        for (int64_t c = 0; c < nchunk; ++c) acc += dApart[(size_t)c * ND + i];
        const int n = (int)(i / D), d = (int)(i % D);
        dA[(size_t)d * NS + n] = acc;
    }
    if (dD && i < D) {
        float acc = 0.0f;
        for (int64_t c = 0; c < nchunk; ++c) acc += dDpart[(size_t)c * D + i];
        dD[i] = acc;
    }
}

template <int NS>
__global__ __launch_bounds__(256) void k_scan_bwd_reduce_bc(const float* __restrict__ dBC, int64_t ngroup,
                                                            int64_t T_, float* __restrict__ dB,
                                                            float* __restrict__ dC) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // t*2NS + j
    if (i >= T_ * 2 * NS) return;
    float acc = 0.0f;
    for (int64_t gi = 0; gi < ngroup; ++gi) acc += dBC[(size_t)gi * T_ * 2 * NS + i];
    const int64_t t = i / (2 * NS);
    const int j = (int)(i % (2 * NS));
    if (j < NS) dB[t * NS + j] = acc;
    else dC[t * NS + (j - NS)] = acc;
}

template <typename T, int NS>
static int scan_bwd_launch(const void* u, const void* delta, const float* A, const void* B, const void* C,
                           const float* Dskip, const void* z, const int32_t* pos, const void* dout, float* ws,
                           void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz, int64_t T_,
                           int D, hipStream_t s) {
    const ScanWs L = scan_ws_layout(T_, D, NS);
    const dim3 grid((unsigned)(L.ngroup * L.nchunk));
    const int64_t ND = (int64_t)NS * D;
    if (L.nchunk > 1) {
        k_scan_bwd_summary<T, NS><<<grid, kWave, 0, s>>>((const T*)delta, A, (const T*)C, (const T*)z,
                                                         (const T*)dout, pos, ws + L.Pr, ws + L.Sr, T_, D);
        SSMP_LAUNCH_CHECK();
    }
    k_scan_bwd_carry<NS><<<(unsigned)((ND + 255) / 256), 256, 0, s>>>(ws + L.Pr, ws + L.Sr, pos, ws + L.cin, D,
                                                                      L.nchunk);
    SSMP_LAUNCH_CHECK();
    BwdArgs<T, NS> a;
    a.u = (const T*)u; a.delta = (const T*)delta; a.A = A; a.B = (const T*)B; a.C = (const T*)C; a.Dskip = Dskip;
    a.z = (const T*)z; a.dout = (const T*)dout; a.pos = pos; a.ckpt = ws + L.ckpt; a.cin = ws + L.cin;
    a.du = (T*)du; a.ddelta = (T*)ddelta; a.dz = (T*)dz; a.dApart = ws + L.dApart; a.dDpart = ws + L.dDpart;
    a.dBC = ws + L.dBC; a.T_ = T_; a.D = D;
    k_scan_bwd_main<T, NS><<<grid, kWave, 0, s>>>(a);
    SSMP_LAUNCH_CHECK();
    const int64_t nrp = ND > D ? ND : D;
    k_scan_bwd_reduce_params<NS><<<(unsigned)((nrp + 255) / 256), 256, 0, s>>>(ws + L.dApart, ws + L.dDpart,
                                                                               L.nchunk, D, dA, dD);
    SSMP_LAUNCH_CHECK();
    k_scan_bwd_reduce_bc<NS><<<(unsigned)((T_ * 2 * NS + 255) / 256), 256, 0, s>>>(ws + L.dBC, L.ngroup, T_, dB,
                                                                                   dC);
    SSMP_LAUNCH_CHECK();
    return SSMP_OK;
}

template <typename T>
static int scan_bwd_dispatch(int N, const void* u, const void* delta, const float* A, const void* B, const void* C,
                             const float* Dskip, const void* z, const int32_t* pos, const void* dout, float* ws,
                             void* du, void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                             int64_t T_, int D, hipStream_t s) {
#define SSMP_BWD_CASE(NV)                                                                                         \
    case NV:                                                                                                      \
        return scan_bwd_launch<T, NV>(u, delta, A, B, C, Dskip, z, pos, dout, ws, du, ddelta, dA, dB, dC, dD, dz, \
                                      T_, D, s);
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

extern "C" int selective_scan_pack_bwd(const void* u, const void* delta, const float* A, const void* B,
                                       const void* C, const float* Dskip, const void* z, const int32_t* pos,
                                       const void* dout, void* workspace, size_t workspace_bytes, void* du,
                                       void* ddelta, float* dA, float* dB, float* dC, float* dD, void* dz,
                                       int64_t T, int32_t D, int32_t N, int32_t dtype, void* stream) {
    using namespace ssmp;
    int st = scan_check_args(T, D, N, dtype);
    if (st) return st;
    if (!A || !dA) return SSMP_ERR_NULL;
    if ((Dskip == nullptr) != (dD == nullptr)) return SSMP_ERR_NULL;
    if ((z == nullptr) != (dz == nullptr)) return SSMP_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        if (hipMemsetAsync(dA, 0, sizeof(float) * (size_t)D * N, s) != hipSuccess) return SSMP_ERR_HIP;
        if (dD && hipMemsetAsync(dD, 0, sizeof(float) * (size_t)D, s) != hipSuccess) return SSMP_ERR_HIP;
        return SSMP_OK;
    }
    if (!u || !delta || !B || !C || !pos || !dout || !du || !ddelta || !dB || !dC) return SSMP_ERR_NULL;
    if (!workspace || workspace_bytes < selective_scan_pack_workspace_bytes(T, D, N)) return SSMP_ERR_WORKSPACE;
    float* ws = static_cast<float*>(workspace);
    return dtype == SSMP_BF16 ? scan_bwd_dispatch<uint16_t>(N, u, delta, A, B, C, Dskip, z, pos, dout, ws, du,
                                                            ddelta, dA, dB, dC, dD, dz, T, D, s)
                              : scan_bwd_dispatch<float>(N, u, delta, A, B, C, Dskip, z, pos, dout, ws, du, ddelta,
                                                         dA, dB, dC, dD, dz, T, D, s);
}
