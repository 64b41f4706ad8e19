// Shared tiling, workspace layout and staging helpers of the selective-scan
// kernels.
#pragma once

#include "common.h"

namespace ssmp {

// Time tiling. A chunk of lc tokens is the unit of time parallelism: one wave
// walks it serially for a group of channels, and chunks are joined by the
// affine carry h_out = P h_in + S (P = 0 once the chunk holds a head). Every
// chunk whose successor continues a sequence costs a summary pass, so chunks
// are as long as the grid allows: the longest power of two (64 .. 2048 tokens)
// that still gives kMinWaves waves. The backward restarts every kCK-token
// block from the state entering it, which the forward keeps (every kCK-th
// token, or every kMinCK-th) or the backward replays, and replays the block
// with its states in registers. Kept every kCK tokens, checkpoints cost 8 B
// of HBM per (t, d) each way and spare the backward a second replay pass.
constexpr int kCK = 8;
constexpr int kMinCK = 4;  // the shortest interval the forward keeps
constexpr int kBB = 16;
constexpr int kLCMin = 64, kLCMax = 2048;
constexpr int64_t kMinWaves = 8192;  // eight per SIMD on 256 CUs: enough to hide load latency
static_assert(kCK % kMinCK == 0 && kLCMin % kBB == 0 && kLCMin % kCK == 0, "tiling");

// waves per backward workgroup: each holds min(N, 4) of the states of the
// workgroup's channels
inline int bwd_waves(int N) { return N / (N < 4 ? N : 4); }
// channels per lane of the backward's main pass (a workgroup covers kBwdCl * 64
// channels)
constexpr int kBwdCl = 1;

inline int scan_chunk_len(int64_t T, int D, int chw) {
    const int64_t ng = (D + chw - 1) / chw;
    int lc = kLCMax;
    while (lc > kLCMin && ng * ((T + lc - 1) / lc) < kMinWaves) lc >>= 1;
    return lc;
}
inline int fwd_chunk_len(int64_t T, int D) { return scan_chunk_len(T, D, kWave); }
inline int bwd_chunk_len(int64_t T, int D, int N) { return scan_chunk_len(T, D, kBwdCl * kWave / bwd_waves(N)); }
// The backward's reverse-carry summaries run over sub-chunks of the main
// kernel's chunks (down to kLCMin tokens): a summary wave's work depends on
// where the heads fall, and more, shorter waves even it out across the SIMDs.
constexpr int kBwdSumSplit = 4;
inline int bwd_sum_len(int64_t T, int D, int N) {
    const int ls = bwd_chunk_len(T, D, N) / kBwdSumSplit;
    return ls < kLCMin ? kLCMin : ls;
}
// A reverse summary of the sub-chunk starting at token t0 (position p0) is
// used only if its sequence started before the start of its main chunk
// (ls << logR tokens): then the carry it forms reaches that chunk's boundary.
__device__ __forceinline__ bool bwd_sum_needed(int32_t p0, int64_t t0, int logR, int ls) {
    const int64_t lc = (int64_t)ls << logR;
    return (int64_t)p0 > t0 % lc;
}

// Optional element-wise neighbours of the scan, applied where the scan reads
// its inputs: the step is softplus(delta + bias[d]) (softplus set) or
// delta + bias[d] (bias may be null), and the gate is silu(z) + gate_floor.
//
// Sequences may also start from a given state and hand on their last one
// (sequences cut at a pack end continue in the next pack): h0 is the state
// before each sequence's first token, hT the state after its last, both
// (nseq, D, N) fp32 with element (s, d, n) at (s*D + d)*N + n; the backward
// takes dhT (the loss gradient with respect to hT) and returns dh0. Null
// pointers switch each part off (h0 and dhT then count as zero). cu is the
// device cu_seqlens, used to name the sequence of a head or end token.
struct ScanOpts {
    const float* delta_bias;
    int softplus;
    float gate_floor;
    const int32_t* cu = nullptr;
    int nseq = 0;
    const float* h0 = nullptr;
    float* hT = nullptr;
    const float* dhT = nullptr;
    float* dh0 = nullptr;
};

// A checkpoint slot holds the states of every channel in groups of four
// ([n/4][d][4] for d_state a multiple of 4, else [n][d]): a wave's 16-byte
// stores of one group cover 1 KiB of contiguous memory, and a lane loads its
// states 16 bytes at a time. Checkpoints are written once by the forward and
// read once by the backward, so both go through non-temporal accesses and
// leave the L2 to the inputs the other waves of the chunk share.
typedef float nf4 __attribute__((ext_vector_type(4)));
template <int NS>
__device__ __forceinline__ size_t ck_index(int d, int n, int D) {
    if constexpr (NS % 4 == 0) return (((size_t)(n >> 2) * D + d) << 2) + (n & 3);
    else return (size_t)n * D + d;
}
// Non-temporal stores through buffer resources over the slot's rows: a lane
// past D (d >= D) lands past its row's end, which the hardware drops, so
// callers need no per-lane branch.
template <int NS>
__device__ __forceinline__ void ck_store(float* __restrict__ slot, int d, int D, const float (&h)[NS]) {
    if constexpr (NS % 4 == 0) {
#pragma unroll
        for (int j = 0; j < NS / 4; ++j) {
            const auto r = bytes_rsrc(slot + (size_t)j * D * 4, (uint32_t)D * 16u);
            const nf4 v = {h[4 * j], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) uint32_t, v),
                                                   r, (int)((uint32_t)d * 16u), 0, kBufNT);
        }
    } else {
#pragma unroll
        for (int n = 0; n < NS; ++n)
            Elt<float>::st_rsrc<kBufNT>(bytes_rsrc(slot + (size_t)n * D, (uint32_t)D * 4u), (uint32_t)d * 4u, h[n]);
    }
}
// states n0 .. n0+NH-1 of channel d (zero when `on` is false)
template <int NS, int NH>
__device__ __forceinline__ void ck_load(const float* __restrict__ slot, int d, int D, int n0, bool on,
                                           float (&h)[NH]) {
    if (!on) {
#pragma unroll
        for (int i = 0; i < NH; ++i) h[i] = 0.0f;
    } else if constexpr (NS % 4 == 0 && NH % 4 == 0) {
#pragma unroll
        for (int j = 0; j < NH / 4; ++j) {
            const nf4 v =
                __builtin_nontemporal_load(reinterpret_cast<const nf4*>(slot) + (size_t)((n0 >> 2) + j) * D + d);
            h[4 * j] = v.x; h[4 * j + 1] = v.y; h[4 * j + 2] = v.z; h[4 * j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NH; ++i) h[i] = slot[ck_index<NS>(d, n0 + i, D)];
    }
}

// Sequence of token t: the largest s with cu[s] <= t (zero-length sequences
// sharing that start come before it). Wave-uniform: every lane of a wave asks
// about the same token, and it runs only at heads and ends. For any cu the
// result stays in [0, nseq-1].
__device__ __forceinline__ int seq_of(const int32_t* __restrict__ cu, int nseq, int64_t t) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Sequences with no tokens hand on their initial state (or its gradient)
// unchanged: dst[s] = src ? src[s] : 0 for every s with cu[s] == cu[s+1].
// One thread per (s, d, n); other sequences are left to the scan kernels.
template <int kUnused = 0>
__global__ __launch_bounds__(256) void k_empty_seq_states(const int32_t* __restrict__ cu, int nseq, int64_t DN,
                                                          const float* __restrict__ src, float* __restrict__ dst) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)nseq * DN) return;
    const int s = (int)(i / DN);
    if (cu[s] == cu[s + 1]) dst[i] = src ? src[i] : 0.0f;
}

// softplus(v) = max(v, 0) + log1p(e) with e = exp(-|v|) in (0, 1]. With
// w = 1 + e rounded and c = e - (w - 1) its rounding error, log1p(e) =
// log(w) + c / w to first order; c alone instead of c / w is off by c e / w,
// under one ulp of log1p(e) >= e ln 2 (when e is below w's ulp, w = 1 and
// the sum is e exactly). One v_exp and one v_log, no division.
__device__ __forceinline__ float softplus_f(float v) {
    const float e = exp2_fast(-__builtin_fabsf(v) * kLog2e);
    const float w = 1.0f + e;
    return __builtin_fmaxf(v, 0.0f) + __builtin_fmaf(__builtin_amdgcn_logf(w), kLn2, e - (w - 1.0f));
}
// The same value and its derivative sigmoid(v): 1/w for v >= 0, e/w below.
__device__ __forceinline__ float softplus_f(float v, float& slope) {
    const float e = exp2_fast(-__builtin_fabsf(v) * kLog2e);
    const float w = 1.0f + e;
    slope = (v >= 0.0f ? 1.0f : e) * __builtin_amdgcn_rcpf(w);
    return __builtin_fmaxf(v, 0.0f) + __builtin_fmaf(__builtin_amdgcn_logf(w), kLn2, e - (w - 1.0f));
}

// The step map of one channel. Off (no bias, no softplus) it is the identity,
// and every call site tests `on` first: a wave-uniform branch.
struct StepMap {
    float bias;
    bool sp;
    bool on;
    __device__ __forceinline__ float eff(float raw) const {
        const float v = raw + bias;
        return sp ? softplus_f(v) : v;
    }
    // the step and its derivative with respect to raw
    __device__ __forceinline__ float eff(float raw, float& slope) const {
        const float v = raw + bias;
        float s = 1.0f;
        const float m = sp ? softplus_f(v, s) : v;
        slope = s;
        return m;
    }
};
__device__ __forceinline__ StepMap step_map(const ScanOpts& o, int d) {
    StepMap m;
    m.bias = o.delta_bias ? o.delta_bias[d] : 0.0f;
    m.sp = o.softplus != 0;
    m.on = o.delta_bias != nullptr || o.softplus != 0;
    return m;
}

// Checkpoint intervals. The forward may keep the state entering every ci-th
// token for the backward (ci a power of two in [kMinCK, kLCMax]), or none (ci
// = 0). The backward restarts every kCK-token block from such a state: with
// ci dividing kCK it reads the kept ones, otherwise it first replays the
// forward's recurrence from them (from the chunk states of a fresh summary
// pass for ci = 0) into dense checkpoints of its own, kCK tokens apart.
inline bool ck_interval_ok(int ci) {
    return ci == 0 || (ci >= kMinCK && ci <= kLCMax && (ci & (ci - 1)) == 0);
}
inline bool ck_direct(int ci) { return ci != 0 && kCK % ci == 0; }
inline size_t ws_up(size_t v) { return (v + 63) & ~size_t(63); }  // 256-byte aligned regions
// floats the forward keeps for the backward: [ceil(T/ci)][N/4][D][4]
inline size_t saved_floats(int64_t T, int D, int N, int ci) {
    return ci ? ws_up((size_t)((T + ci - 1) / ci) * (size_t)N * D) : 0;
}

// The scratch of one pass (offsets in floats from its base). Nothing in it
// outlives the call.
struct ScanWs {
    int64_t nck;      // dense checkpoint slots: slot j holds the state entering token j*kCK
    int64_t nfchunk;  // forward chunks
    int64_t nbchunk;  // backward chunks
    int64_t nsum;     // backward summary sub-chunks
    int64_t ngroup;   // channel groups of 64
    size_t bc;        // [T][2N]          fp32 copy of the B and C rows (each pass makes its own)
    size_t P, S;      // forward: P [nfchunk][D] sum of delta (NaN: cut by a head), S [nfchunk][N][D] local end state
    size_t hin;       // [nfchunk][N/4][D][4] forward: state entering each chunk
    size_t dense;     // [nck][N/4][D][4] backward unless ck_direct(ci): replayed checkpoints
    size_t Pr, Sr;    // backward, per summary sub-chunk: Pr [nsum][D] as P, Sr [nsum][N][D] reverse carry
    size_t cin;       // [nbchunk][N][D]  backward: carry entering each chunk from the right
    size_t dApart;    // [nbchunk][N][D]
    size_t dDpart;    // [nbchunk][D]
    size_t dbpart;    // [nbchunk][D]     backward: step-bias gradient partials
    size_t dBC;       // [<= ceil(D/64)][T][2N]  per channel-group partial sums of dB, dC
    size_t sink;      // [64] target of stores by lanes with nothing to store (kept branch-free)
    size_t fwd_total; // floats the forward uses
    size_t bwd_total; // floats the backward uses with checkpoint interval ci
};

// The forward's regions come first; the backward with ci = 0 reruns the
// forward's summary and carry passes in them before its own.
inline ScanWs scan_ws_layout(int64_t T, int D, int N, int ci) {
    ScanWs w{};
    w.nck = (T + kCK - 1) / kCK;
    const int64_t lf = fwd_chunk_len(T, D), lb = bwd_chunk_len(T, D, N);
    w.nfchunk = (T + lf - 1) / lf;
    w.nbchunk = (T + lb - 1) / lb;
    const int64_t ls = bwd_sum_len(T, D, N);
    w.nsum = (T + ls - 1) / ls;
    w.ngroup = (D + kWave - 1) / kWave;
    const size_t ND = (size_t)N * D;
    size_t off = 0;
    w.bc = off; off = ws_up(off + (size_t)T * 2 * N);
    const size_t after_bc = off;
    w.P = off; off = ws_up(off + (size_t)w.nfchunk * D);
    w.S = off; off = ws_up(off + (size_t)w.nfchunk * ND);
    w.hin = off; off = ws_up(off + (size_t)w.nfchunk * ND);
    w.fwd_total = off;
    off = (ci == 0) ? w.fwd_total : after_bc;
    if (!ck_direct(ci)) { w.dense = off; off = ws_up(off + (size_t)w.nck * ND); }
    w.Pr = off; off = ws_up(off + (size_t)w.nsum * D);
    w.Sr = off; off = ws_up(off + (size_t)w.nsum * ND);
    w.cin = off; off = ws_up(off + (size_t)w.nbchunk * ND);
    w.dApart = off; off = ws_up(off + (size_t)w.nbchunk * ND);
    w.dDpart = off; off = ws_up(off + (size_t)w.nbchunk * D);
    w.dbpart = off; off = ws_up(off + (size_t)w.nbchunk * D);
    w.dBC = off; off = ws_up(off + (size_t)((D + kWave - 1) / kWave) * (size_t)T * 2 * N);
    w.sink = off; off = ws_up(off + 64);
    w.bwd_total = off;
    return w;
}

// Dense checkpoints for the backward (scratch + L.dense), replayed from the
// forward's kept states at interval ci, or for ci = 0 from the chunk states of
// a fresh forward summary pass. Needs the fp32 B/C rows at scratch + L.bc.
// Defined with the forward kernels.
int scan_dense_ckpt(int N, bool bf16, const void* u, const void* delta, const float* A, const int32_t* pos,
                    const float* saved, int ci, float* scratch, int64_t T, int D, const ScanOpts& o, hipStream_t s);

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
    if (((T + kLCMin - 1) / kLCMin) * ((D + 31) / 32) >= (int64_t(1) << 31)) return SSMP_ERR_SHAPE;
    if ((T * (int64_t)D) >= (int64_t(1) << 40)) return SSMP_ERR_SHAPE;
    if (!(N == 1 || N == 2 || N == 4 || N == 8 || N == 16)) return SSMP_ERR_UNSUPPORTED;
    if (dtype != SSMP_F32 && dtype != SSMP_BF16) return SSMP_ERR_UNSUPPORTED;
    return SSMP_OK;
}

// B and C rows of every token as fp32, interleaved: bc[t] = [B_t (N), C_t (N)],
// so one wave-uniform scalar load brings both rows of a token.
template <typename T, int NS>
__global__ __launch_bounds__(256) void k_bc_to_f32(const T* __restrict__ B, const T* __restrict__ C,
                                                  float* __restrict__ bc, int64_t T_) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // t*2NS + j
    if (i >= T_ * 2 * NS) return;
    const int64_t t = i / (2 * NS);
    const int j = (int)(i % (2 * NS));
    bc[i] = (j < NS) ? Elt<T>::ld(B, (size_t)t * NS + j) : Elt<T>::ld(C, (size_t)t * NS + (j - NS));
}

template <int NS>
__device__ __forceinline__ void load_bc(const float* __restrict__ bc, int64_t t, float (&Bv)[NS], float (&Cv)[NS]) {
    const float* __restrict__ row = bc + (size_t)t * 2 * NS;
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        Bv[n] = row[n];
        Cv[n] = row[NS + n];
    }
}

// Head flags of the BT tokens of a block as a wave-uniform bit mask (bit k:
// token tb+k starts a sequence). Lanes k < BT each read one position.
template <int BT = kBB>
__device__ __forceinline__ uint32_t block_heads(const int32_t* __restrict__ pos, int64_t tb, int64_t T_, int lane) {
    const int64_t t = tb + lane;
    const bool f = (lane < BT) && (t < T_) && pos[t] == 0;
    return (uint32_t)__ballot(f);
}

// End flags of the BT tokens of a block (bit k: token tb+k is the last of its
// sequence, i.e. tb+k+1 is a head or the end of the pack). Lanes k < BT each
// read one position, one token further on than block_heads.
template <int BT = kBB>
__device__ __forceinline__ uint32_t block_ends(const int32_t* __restrict__ pos, int64_t tb, int64_t T_, int lane) {
    const int64_t t = tb + lane;
    const bool f = (lane < BT) && (t < T_) && (t + 1 == T_ || pos[t + 1] == 0);
    return (uint32_t)__ballot(f);
}

// Reset of the state at a head token. Heads are rare, so this stays a real
// (wave-uniform) branch: the empty volatile asm keeps the compiler from
// turning it into a select on every state of every token.
template <int NS>
__device__ __forceinline__ void reset_if(bool head, float (&h)[NS]) {
    if (head) {
        asm volatile("");
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = 0.0f;
    }
}

// Staging of R per-lane (T, D) inputs for one BT-token block of a 64-channel
// group into LDS, laid out [r][k][64]. With 16-byte aligned rows (D a
// multiple of 16 / sizeof(T)) the block is fetched into registers with
// 16-byte loads one block ahead, and committed to LDS when the block starts;
// otherwise each lane copies its own elements at commit time.
template <typename T, int R, int BT = kBB, int CW = kWave>
struct Stager {
    static constexpr int EPV = 16 / (int)sizeof(T);      // elements per 16-byte piece
    static constexpr int PPR = CW / EPV;                  // pieces per row of CW channels
    static constexpr int NP = R * BT * PPR / kWave;       // pieces per lane
    static_assert((R * BT * PPR) % kWave == 0, "staging shape");
    static constexpr int kElems = R * BT * CW;            // LDS elements of one block
    uint4 reg[NP];

    __device__ __forceinline__ void fetch(const T* const (&src)[R], int64_t tb, int64_t T_, int D, int g, int lane,
                                          bool vec) {
        if (!vec) return;
        if (tb + BT <= T_ && (g + 1) * CW <= D) {
            // whole block inside the tensor: no per-piece bounds
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int q = p * kWave + lane;
                const int row = q / PPR, j = q % PPR;
                const int r = row / BT, k = row % BT;
                reg[p] = *reinterpret_cast<const uint4*>(src[r] + (size_t)(tb + k) * D + g * CW + j * EPV);
            }
            return;
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int q = p * kWave + lane;
            const int row = q / PPR, j = q % PPR;
            const int r = row / BT, k = row % BT;
            const int64_t t = tb + k;
            const int ch = g * CW + j * EPV;
            // pieces outside the tensor stage zeros, so lanes past D only see finite inputs
            reg[p] = (t < T_ && ch < D) ? *reinterpret_cast<const uint4*>(src[r] + (size_t)t * D + ch)
                                        : make_uint4(0u, 0u, 0u, 0u);
        }
    }

    __device__ __forceinline__ void commit(T* lds, const T* const (&src)[R], int64_t tb, int64_t T_, int D, int g,
                                           int lane, bool vec) {
        if (vec) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int q = p * kWave + lane;
                const int row = q / PPR, j = q % PPR;
                *reinterpret_cast<uint4*>(lds + row * CW + j * EPV) = reg[p];
            }
        } else if (lane < CW) {
            const int d = g * CW + lane;
#pragma unroll
            for (int r = 0; r < R; ++r)
                for (int k = 0; k < BT; ++k) {
                    const int64_t t = tb + k;
                    lds[(r * BT + k) * CW + lane] = (t < T_ && d < D) ? src[r][(size_t)t * D + d] : T(0);
                }
        }
    }

    // element (r, k) of channel c (0 <= c < CW) of the committed block
    static __device__ __forceinline__ float get(const T* lds, int r, int k, int c) {
        return Elt<T>::ld(lds, (size_t)(r * BT + k) * CW + c);
    }
};

// Tile of the flat grid over (chunk, group of CW channels), group fastest.
template <int CW>
__device__ __forceinline__ Tile tile_of_w(int D) {
    const unsigned ng = (unsigned)((D + CW - 1) / CW);
    return Tile{(int)(blockIdx.x % ng), (int64_t)(blockIdx.x / ng)};
}

template <typename T>
inline bool stage_vec_ok(int D, std::initializer_list<const void*> ptrs) {
    if (D % (16 / (int)sizeof(T)) != 0) return false;
    for (const void* p : ptrs)
        if (p && (reinterpret_cast<uintptr_t>(p) & 15u)) return false;
    return true;
}

}  // namespace ssmp
