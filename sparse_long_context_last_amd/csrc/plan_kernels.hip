// FlexPrefill steps 1 and 2 on gfx950: query-aware sparse pattern
// determination and cumulative-attention index selection (abstract items 1-2
// on the OpenReview / codewithpapers pages; "Approach" paragraph and ablation
// table of the atlas.scime.ai summary page).
//
// Every kernel here computes in the library's canonical arithmetic: each
// float32 / float64 rounding point and every reduction order is fixed (no
// contraction into fused multiply-adds unless a product is exact, sequential
// sums in ascending index order, exp2 / ln from fixed series), and the gamma
// test is done on integers.  The resulting pattern choices and block lists
// are therefore bit-reproducible across runs and launch geometries.
#pragma clang fp contract(off)

#include <cstring>

#include "fp_common.h"
#include "fp_launch.h"

namespace fp {

// ---------------------------------------------------------------------------
// canonical elementary functions
// ---------------------------------------------------------------------------

// 2^x for x <= 0: +0 below -100; else n = rint(x), f = x - n, Horner in f of
// the degree-7 Taylor series of 2^f (every product and sum rounded), times 2^n.
__device__ __forceinline__ float exp2_c(float x, const Canon& K) {
    if (!(x >= -100.0f)) return 0.0f;
    float n = rintf(x);
    float f = x - n;
    float p = K.e2[7];
#pragma unroll
    for (int i = 6; i >= 0; --i) {
        p = p * f;
        p = p + K.e2[i];
    }
    return ldexpf(p, (int)n);
}

// ln x for x > 0 in binary64: x = m 2^e with m in [sqrt(1/2), sqrt(2)),
// ln m = 2 artanh z, z = (m - 1)/(m + 1), series truncated after z^21.
__device__ __forceinline__ double ln_c(double x, const Canon& K) {
    int e;
    double m = frexp(x, &e);
    if (m < K.sqrt_half) {
        m = m * 2.0;
        e = e - 1;
    }
    double z = (m - 1.0) / (m + 1.0);
    double w = z * z;
    double s = K.lnc[10];
#pragma unroll
    for (int i = 9; i >= 0; --i) {
        s = s * w;
        s = s + K.lnc[i];
    }
    double a = (double)e * K.ln2;
    double b = (2.0 * z) * s;
    return a + b;
}

// Fixed-point mass of a value: rint(x * 2^32) (x >= 0, x <= 2^31).
__device__ __forceinline__ unsigned long long fixed_u(float x) {
    return (unsigned long long)rintf(x * 4294967296.0f);
}

// Ordering key: value descending, then index ascending <=> key ascending.
__device__ __forceinline__ unsigned long long order_key(float x, long long idx, int ibits) {
    unsigned int inv = 0x7FFFFFFFu - __float_as_uint(x);
    return ((unsigned long long)inv << ibits) | (unsigned long long)idx;
}

// Load n consecutive elements (16-byte aligned) widened to fp32; zeros if !ok.
template <typename T, int n> __device__ __forceinline__ void load_row_f32(const T* p, bool ok, float* out);
template <> __device__ __forceinline__ void load_row_f32<bf16_t, kScoreDSConst>(const bf16_t* p, bool ok, float* out) {
#pragma unroll
    for (int v = 0; v < kScoreDSConst / 8; ++v) {
        uint4 w = ok ? reinterpret_cast<const uint4*>(p)[v] : make_uint4(0, 0, 0, 0);
        const unsigned int ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[v * 8 + 2 * e] = __uint_as_float(ws[e] << 16);
            out[v * 8 + 2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
        }
    }
}
template <> __device__ __forceinline__ void load_row_f32<float, kScoreDSConst>(const float* p, bool ok, float* out) {
#pragma unroll
    for (int v = 0; v < kScoreDSConst / 4; ++v) {
        float4 w = ok ? reinterpret_cast<const float4*>(p)[v] : make_float4(0.f, 0.f, 0.f, 0.f);
        out[v * 4] = w.x; out[v * 4 + 1] = w.y; out[v * 4 + 2] = w.z; out[v * 4 + 3] = w.w;
    }
}

template <typename T> struct MulAdd;
// bf16 inputs: the product of two bf16 values is exact in fp32, so one fused
// multiply-add rounds exactly like the product-then-sum of the definition.
template <> struct MulAdd<bf16_t> {
    static __device__ __forceinline__ float step(float acc, float a, float b) {
        return __builtin_fmaf(a, b, acc);
    }
};
template <> struct MulAdd<float> {
    static __device__ __forceinline__ float step(float acc, float a, float b) {
        float p = a * b;
        return acc + p;
    }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// ---------------------------------------------------------------------------
// K1: block means ("block-pooled" queries and keys)
// out[head][kb][t] = (sum_r x[kb*bs + r][t], r ascending) / rows(kb), where
// rows(kb) = bs except for a partial last block (for a full block the
// division is the exact scaling by 1/bs).
// 256 threads = 16 key blocks x 16 column groups of 8; each thread keeps 8
// sequential sums and reads 16-byte (bf16) / 32-byte (fp32) row pieces.
// grid (ceil(nb / 16), heads), head = b * H + h.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float* v);
template <> __device__ __forceinline__ void load8_f32<bf16_t>(const bf16_t* p, float* v) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const unsigned int ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        v[2 * e] = __uint_as_float(ws[e] << 16);
        v[2 * e + 1] = __uint_as_float(ws[e] & 0xFFFF0000u);
    }
}
template <> __device__ __forceinline__ void load8_f32<float>(const float* p, float* v) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void k_pool(const T* __restrict__ x, TokStride xs, int H,
                                              float* __restrict__ out, int L, int bs) {
    constexpr int TPR = D / 8, RPW = 256 / TPR;   // threads per block row, block rows per workgroup
    const int tid = threadIdx.x, cg = tid % TPR;
    const int kb = blockIdx.x * RPW + tid / TPR, head = blockIdx.y;
    const int nb = (L + bs - 1) / bs;
    if (kb >= nb) return;
    const int rows = min(bs, L - kb * bs);
    const T* src = x + (size_t)(head / H) * xs.bst + (size_t)(head % H) * xs.hs + (size_t)kb * bs * xs.rs + 8 * cg;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll 8
    for (int r = 0; r < rows; ++r) {
        float v[8];
        load8_f32<T>(src + (size_t)r * xs.rs, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = acc[e] + v[e];
    }
    float* dst = out + ((size_t)head * nb + kb) * D + 8 * cg;
    const float fr = (float)rows;
    float4 lo, hi;
    lo.x = acc[0] / fr; lo.y = acc[1] / fr; lo.z = acc[2] / fr; lo.w = acc[3] / fr;
    hi.x = acc[4] / fr; hi.y = acc[5] / fr; hi.z = acc[6] / fr; hi.w = acc[7] / fr;
    reinterpret_cast<float4*>(dst)[0] = lo;
    reinterpret_cast<float4*>(dst)[1] = hi;
}

// ---------------------------------------------------------------------------
// K2: exact scores of the last query block against every key.
// s2[bh][i][j] = fp32(sum_t q[L-BS+i][t] * k[j][t]) * C, t ascending; plus the
// per-(row, 256-key chunk) maxima over causal keys (j <= L-BS+i).  Rows with
// L-BS+i < 0 (a sequence shorter than one block) do not exist: their maxima
// stay -inf and later kernels skip them.
// (fp32 inputs; bf16 ones run k_scores_mfma below.)
// Register-blocked VALU product: 256 threads, tile BS queries x 256 keys, each
// thread owns BS/16 queries x 16 keys; d staged through LDS in slices of 32
// (the query slices from the transposed copy k_qt writes).
// ---------------------------------------------------------------------------
constexpr int kScoreTK = 256;
constexpr int kScoreDS = kScoreDSConst;

// The last block's queries, widened to fp32 and transposed once per call:
// qt[bh][t][i] = q[L-BS+i][t] (0 for rows that do not exist), so that every
// score workgroup stages its query slices with contiguous 16-byte loads.
template <typename T, int BS, int D>
__global__ __launch_bounds__(BS) void k_qt(const T* __restrict__ q, TokStride qs, float* __restrict__ qt, int L,
                                           int Hq) {
    const int i = threadIdx.x, t0 = 8 * blockIdx.x, bh = blockIdx.y;
    const int b = bh / Hq, h = bh % Hq;
    const int pos = L - BS + i;
    float v[8];
    if (pos >= 0) {
        load8_f32<T>(q + (size_t)b * qs.bst + (size_t)h * qs.hs + (size_t)pos * qs.rs + t0, v);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) qt[((size_t)bh * D + t0 + e) * BS + i] = v[e];
}

// Built for three waves per SIMD (at most 168 registers), which measured
// faster than two waves with more room.
template <typename T, int BS, int D>
__global__ __launch_bounds__(256, 3) void k_scores(const float* __restrict__ qt, const T* __restrict__ k,
                                                TokStride ks, float* __restrict__ s2,
                                                float* __restrict__ pmax, int L, int NS, int Hq, int group,
                                                float C) {
    constexpr int TK = kScoreTK, DS = kScoreDS, MR = BS / 16;
    static_assert(D % DS == 0, "d slices");
    __shared__ __attribute__((aligned(16))) float Qs[DS][BS + 4];
    __shared__ __attribute__((aligned(16))) float Ks[DS][TK + 4];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int b = bh / Hq, h = bh % Hq;
    const float* qth = qt + (size_t)bh * D * BS;
    const int j0 = chunk * TK;
    const T* kbase = k + (size_t)b * ks.bst + (size_t)(h / group) * ks.hs;
    const bool key_ok = (j0 + tid) < L;

    float acc[MR][16];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int n = 0; n < 16; ++n) acc[m][n] = 0.0f;

    for (int t0 = 0; t0 < D; t0 += DS) {
        // Q slice, transposed: Qs[tt][i]
        for (int e4 = tid; e4 < BS * DS / 4; e4 += 256) {
            const int tt = e4 / (BS / 4), i = 4 * (e4 % (BS / 4));
            *reinterpret_cast<float4*>(&Qs[tt][i]) = *reinterpret_cast<const float4*>(qth + (size_t)(t0 + tt) * BS + i);
        }
        // K slice, transposed: thread tid owns key j0 + tid
        {
            float kv[DS];
            load_row_f32<T, DS>(kbase + (size_t)(key_ok ? j0 + tid : 0) * ks.rs + t0, key_ok, kv);
#pragma unroll
            for (int tt = 0; tt < DS; ++tt) Ks[tt][tid] = kv[tt];
        }
        __syncthreads();
#pragma unroll 4
        for (int tt = 0; tt < DS; ++tt) {
            float qv[MR], kv[16];
#pragma unroll
            for (int m4 = 0; m4 < MR; m4 += 4) {
                float4 v = *reinterpret_cast<const float4*>(&Qs[tt][ty * MR + m4]);
                qv[m4] = v.x; qv[m4 + 1] = v.y; qv[m4 + 2] = v.z; qv[m4 + 3] = v.w;
            }
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                float4 v = *reinterpret_cast<const float4*>(&Ks[tt][n * 64 + tx * 4]);
                kv[n * 4] = v.x; kv[n * 4 + 1] = v.y; kv[n * 4 + 2] = v.z; kv[n * 4 + 3] = v.w;
            }
#pragma unroll
            for (int m = 0; m < MR; ++m)
#pragma unroll
                for (int n = 0; n < 16; ++n) acc[m][n] = MulAdd<T>::step(acc[m][n], qv[m], kv[n]);
        }
        __syncthreads();
    }

    const int nchunks = NS / TK;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        const int i = ty * MR + m;
        const int pos = L - BS + i;
        float mx = -INFINITY;
        float* row = s2 + ((size_t)bh * BS + i) * NS;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int j = j0 + n * 64 + tx * 4;
            float4 v;
            v.x = acc[m][n * 4] * C;
            v.y = acc[m][n * 4 + 1] * C;
            v.z = acc[m][n * 4 + 2] * C;
            v.w = acc[m][n * 4 + 3] * C;
            {
                *reinterpret_cast<float4*>(row + j) = v;
                if (j <= pos) mx = fmaxf(mx, v.x);
                if (j + 1 <= pos) mx = fmaxf(mx, v.y);
                if (j + 2 <= pos) mx = fmaxf(mx, v.z);
                if (j + 3 <= pos) mx = fmaxf(mx, v.w);
            }
        }
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        if (tx == 0) pmax[((size_t)bh * nchunks + chunk) * BS + i] = mx;
    }
}

// ---------------------------------------------------------------------------
// K2 for bf16 inputs on the matrix unit.  v_mfma_f32_32x32x2_f32 adds its two
// products to the accumulator one after the other, each add rounded to fp32
// (k index 0 first): measured bit-identical to two fused multiply-adds, k = 0
// then k = 1, over 16.8 M outputs including denormal and signed-zero cases.
// Products of bf16 values are exact in fp32, so a chain of these MFMAs over
// d = (0, 1), (2, 3), ... computes exactly the sequential sum of the
// definition, at twice the fp32 rate of the vector ALU.
// Persistent over key chunks: workgroup g of a head takes the 256-key chunks
// g, g + P, ... (P = gridDim.x), so the block's queries are loaded into
// registers once (wave w: 32 queries, lane l holds q[l % 32][2 t + l / 32],
// t = 0..63).  They are the B operand of the transposed product
// S^T = K Q^T, so every lane ends up with one query's scores, four
// consecutive keys per register group, stored with 16-byte writes.  A step
// covers 128 keys: at block 128 each wave takes all of them (four 32-key
// tiles, four independent accumulator chains), at block 64 two waves share
// the queries and each takes 64 keys.  Key tiles go from global memory
// straight into LDS (buffer loads, 16-byte chunks XOR-swizzled by row),
// double buffered: the next step's tile loads while this step computes.
// Built for two waves per SIMD.  Used for bf16 inputs (fp32 ones keep
// k_scores).
// Same outputs as k_scores: s2 (0 past L) and the per-chunk causal row maxima.
// The bf16 half of a key word is widened with one v_perm_b32 per MFMA, and
// steps whose keys all precede the first query position skip the causal and
// length tests: the vector ALU then issues about a third of the instructions
// of shift/mask/select widening with the tests everywhere, and the kernel
// takes 1.31-1.37 ms on the 128k layer (1.54 ms before; 1.9 ms for k_scores).
// Storing a step's scores during the next step's MFMAs, or two tiles per
// step at three waves per SIMD, ran out of registers (spills) and measured
// slower.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_copy16(const void* base, unsigned voff, void* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000),
        (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

template <int BS, int D>
__global__ __launch_bounds__(256, 2) void k_scores_mfma(const float* __restrict__ qt, const bf16_t* __restrict__ k,
                                                        TokStride ks, float* __restrict__ s2,
                                                        float* __restrict__ pmax, int L, int NS, int Hq, int group,
                                                        float C) {
    typedef float f32x16_t __attribute__((ext_vector_type(16)));
    constexpr int TK = kScoreTK, QG = BS / 32, KG = 4 / QG;
    constexpr int RB = 2 * D, CH = D / 8, RPL = 1024 / RB;   // bytes, 16-byte chunks per key row; rows per 1 KB load
    constexpr int NQ = 4 / KG;                   // 32-key tiles per wave per step
    constexpr int KP = 32 * NQ * KG;             // keys per step (all waves): 128
    constexpr int SPC = TK / KP;                 // steps per 256-key chunk
    constexpr int TILE = KP * D * 2;             // bytes of one step's keys
    constexpr int LOADS = TILE / 1024 / 4;       // 1 KB buffer loads per wave per step
    static_assert(QG * KG == 4 && TK % KP == 0 && LOADS >= 1, "wave layout");
    __shared__ __attribute__((aligned(1024))) unsigned char Kb0[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char Kb1[TILE];
    __shared__ float red[KG][BS];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qg = w % QG, kg = w / QG;
    const int l32 = lane & 31, par = lane >> 5;
    const int bh = blockIdx.y, g = blockIdx.x, P = gridDim.x;
    const int b = bh / Hq, h = bh % Hq;
    const int nchunks = NS / TK;
    const int mych = g < nchunks ? (nchunks - 1 - g) / P + 1 : 0;
    const int nst = mych * SPC;
    if (nst == 0) return;
    const unsigned char* kbase = (const unsigned char*)(k + (size_t)b * ks.bst + (size_t)(h / group) * ks.hs);
    const size_t krs = (size_t)ks.rs * 2;       // bytes per key row

    // queries of this wave: A operand of step t = q[i][2 t + par]
    float qa[D / 2];
    {
        const float* qp = qt + (size_t)bh * D * BS + qg * 32 + l32;
#pragma unroll
        for (int t = 0; t < D / 2; ++t) qa[t] = qp[(size_t)(2 * t + par) * BS];
    }
    // key tile loads: load j of wave w covers rows RPL (w + 4 j) + lane / CH; stored
    // 16-byte chunk lane % CH of a row holds chunk (lane % CH) ^ (row % CH).
    // Rows past L read row L - 1 (finite; their scores are stored as 0).
#define FP_KLOAD(st_, KD_)                                                                                 \
    {                                                                                                      \
        const int key0_ = (g + P * ((st_) / SPC)) * TK + ((st_) % SPC) * KP;                               \
        _Pragma("unroll") for (int j = 0; j < LOADS; ++j) {                                                \
            const int r_ = RPL * (w + 4 * j) + lane / CH;                                                  \
            const int kr_ = min(key0_ + r_, L - 1);                                                        \
            lds_copy16(kbase, (unsigned)((size_t)kr_ * krs + 16 * ((lane % CH) ^ (r_ & (CH - 1)))),        \
                       &KD_[(w + 4 * j) * 1024]);                                                          \
        }                                                                                                  \
    }
    // this lane's key row within the step: kg 128 + 32 q + l32; its 16-byte chunk c sits at c ^ (row % CH)
    const int krow0 = kg * 32 * NQ + l32;
    // byte selector of v_perm_b32 that widens this lane's bf16 half of a 32-bit
    // word to fp32 (bits moved to the top, low half zero): the low half for
    // contraction index 2 t, the high half for 2 t + 1
    const unsigned bsel = par ? 0x03020c0cu : 0x01000c0cu;
    // this lane's query of the transposed product S^T = K Q^T, and its position
    const int qi = qg * 32 + l32, qpos = L - BS + qi;
    float* const srow = s2 + ((size_t)bh * BS + qi) * NS;
    float mx = -INFINITY;
    f32x16_t acc[NQ];

    // one step: MFMAs over the tile in KB_ (keys key0_ ..), then the scores
    // stored and their causal row maxima
#define FP_SSTEP(st_, KB_, KN_)                                                                            \
    {                                                                                                      \
        if ((st_) + 1 < nst) { FP_KLOAD((st_) + 1, KN_); }                                                 \
        const int key0_ = (g + P * ((st_) / SPC)) * TK + ((st_) % SPC) * KP;                               \
        _Pragma("unroll") for (int q = 0; q < NQ; ++q)                                                     \
        _Pragma("unroll") for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;                                   \
        _Pragma("unroll") for (int c = 0; c < D / 8; ++c) {                                                \
            uint4 bv[NQ];                                                                                  \
            _Pragma("unroll") for (int q = 0; q < NQ; ++q) {                                               \
                const int row = krow0 + 32 * q;                                                            \
                bv[q] = *reinterpret_cast<const uint4*>(&KB_[row * RB + 16 * (c ^ (row & (CH - 1)))]);     \
            }                                                                                              \
            _Pragma("unroll") for (int u = 0; u < 4; ++u)                                                  \
            _Pragma("unroll") for (int q = 0; q < NQ; ++q) {                                               \
                const unsigned wd = u == 0 ? bv[q].x : u == 1 ? bv[q].y : u == 2 ? bv[q].z : bv[q].w;      \
                const float kb = __uint_as_float(__builtin_amdgcn_perm(0u, wd, bsel));                     \
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(kb, qa[4 * c + u], acc[q], 0, 0, 0);         \
            }                                                                                              \
        }                                                                                                  \
        /* lane: query qi, keys .. + 32 q + 8 (r / 4) + 4 par + r % 4: four consecutive per store. */    \
        /* A step whose keys all precede the first query position needs neither the causal */            \
        /* nor the length test (uniform branch). */                                                      \
        if (key0_ + KP <= L - BS + 1) {                                                                    \
            _Pragma("unroll") for (int q = 0; q < NQ; ++q)                                                 \
            _Pragma("unroll") for (int g4 = 0; g4 < 4; ++g4) {                                             \
                const int j = key0_ + kg * 32 * NQ + 32 * q + 8 * g4 + 4 * par;                            \
                float4 v_;                                                                                 \
                v_.x = acc[q][4 * g4] * C;                                                                 \
                v_.y = acc[q][4 * g4 + 1] * C;                                                             \
                v_.z = acc[q][4 * g4 + 2] * C;                                                             \
                v_.w = acc[q][4 * g4 + 3] * C;                                                             \
                mx = fmaxf(fmaxf(mx, v_.x), v_.y);                                                         \
                mx = fmaxf(fmaxf(mx, v_.z), v_.w);                                                         \
                *reinterpret_cast<float4*>(srow + j) = v_;                                                 \
            }                                                                                              \
        } else {                                                                                           \
            _Pragma("unroll") for (int q = 0; q < NQ; ++q)                                                 \
            _Pragma("unroll") for (int g4 = 0; g4 < 4; ++g4) {                                             \
                const int j = key0_ + kg * 32 * NQ + 32 * q + 8 * g4 + 4 * par;                            \
                float4 v_;                                                                                 \
                v_.x = acc[q][4 * g4] * C;                                                                 \
                v_.y = acc[q][4 * g4 + 1] * C;                                                             \
                v_.z = acc[q][4 * g4 + 2] * C;                                                             \
                v_.w = acc[q][4 * g4 + 3] * C;                                                             \
                if (j <= qpos) mx = fmaxf(mx, v_.x);                                                       \
                if (j + 1 <= qpos) mx = fmaxf(mx, v_.y);                                                   \
                if (j + 2 <= qpos) mx = fmaxf(mx, v_.z);                                                   \
                if (j + 3 <= qpos) mx = fmaxf(mx, v_.w);                                                   \
                if (j >= L) v_.x = 0.0f;                                                                   \
                if (j + 1 >= L) v_.y = 0.0f;                                                               \
                if (j + 2 >= L) v_.z = 0.0f;                                                               \
                if (j + 3 >= L) v_.w = 0.0f;                                                               \
                *reinterpret_cast<float4*>(srow + j) = v_;                                                 \
            }                                                                                              \
        }                                                                                                  \
        if ((st_) % SPC == SPC - 1) {                                                                      \
            /* chunk done: its row maxima (the other half of the keys sits in lane ^ 32) */                \
            const int chunk_ = g + P * ((st_) / SPC);                                                      \
            const float m_ = fmaxf(mx, __shfl_xor(mx, 32));                                                \
            if (KG == 1) {                                                                                 \
                if (par == 0) pmax[((size_t)bh * nchunks + chunk_) * BS + qi] = m_;                        \
            } else {                                                                                       \
                if (par == 0) red[kg][qi] = m_;                                                            \
                __syncthreads();                                                                           \
                for (int i_ = tid; i_ < BS; i_ += 256) {                                                   \
                    float mm_ = red[0][i_];                                                                \
                    _Pragma("unroll") for (int g2 = 1; g2 < KG; ++g2) mm_ = fmaxf(mm_, red[g2][i_]);       \
                    pmax[((size_t)bh * nchunks + chunk_) * BS + i_] = mm_;                                 \
                }                                                                                          \
            }                                                                                              \
            mx = -INFINITY;                                                                                \
        }                                                                                                  \
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                                   \
        __syncthreads();                                                                                   \
    }

    FP_KLOAD(0, Kb0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
        FP_SSTEP(st, Kb0, Kb1);
        if (st + 1 < nst) FP_SSTEP(st + 1, Kb1, Kb0);
    }
#undef FP_SSTEP
#undef FP_KLOAD
}

// Workgroups per head for k_scores_mfma: about two per CU in all, at most one per chunk.
inline int scores_mfma_groups(int BH, int nchunks) {
    const int want = (2 * 256 + BH - 1) / BH;
    return want < nchunks ? want : nchunks;
}

// ---------------------------------------------------------------------------
// K3a: per last-block row: M = max, e = exp2_c(s - M) (0 for j > pos);
// zpart[kb] = sum over the block's keys ascending; Z = sum of zpart
// over kb ascending; rz = 1 / Z.  One workgroup per (bh, row); the row is
// walked in segments of 4096 keys (32 blocks of 128, 64 of 64) staged
// through LDS (17 KB, so several rows share a CU and one row's loads overlap
// another's arithmetic), where one thread per key block forms its sequential
// sum.  A row that does not exist
// (pos < 0) gets M = Z = rz = 0, so it adds exact zeros downstream.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(256) void k_rowexp(const float* __restrict__ s2, const float* __restrict__ pmax,
                                                float* __restrict__ rowmax, float* __restrict__ rowsum,
                                                float* __restrict__ rz, int L, int NS, Canon K) {
    constexpr int kRowSeg = 4096 / BS;      // blocks per segment: 4096 keys at either block size
    constexpr int SEG = kRowSeg * BS;
    __shared__ float es[kRowSeg][BS + 1];
    __shared__ float zs[kRowSeg];
    __shared__ float red[256];
    const int tid = threadIdx.x;
    const int row = blockIdx.x, bh = blockIdx.y;
    const int nchunks = NS / kScoreTK;
    const int pos = L - BS + row;
    if (pos < 0) {
        if (tid == 0) {
            rowmax[(size_t)bh * BS + row] = 0.0f;
            rowsum[(size_t)bh * BS + row] = 0.0f;
            rz[(size_t)bh * BS + row] = 0.0f;
        }
        return;
    }
    float mx = -INFINITY;
    for (int c = tid; c < nchunks; c += 256) mx = fmaxf(mx, pmax[((size_t)bh * nchunks + c) * BS + row]);
    red[tid] = mx;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] = fmaxf(red[tid], red[tid + s]);
        __syncthreads();
    }
    const float M = red[0];
    const float* srow = s2 + ((size_t)bh * BS + row) * NS;
    // the next segment's loads are in flight while the current one is summed;
    // keys at or past L read key 0 and count as 0
    constexpr int NU = SEG / 1024;
    float4 buf[NU];
#define FP_LOAD_SEG(seg_)                                                                                  \
    _Pragma("unroll") for (int u = 0; u < NU; ++u) {                                                     \
        const int j = (seg_) + u * 1024 + 4 * tid;                                                       \
        buf[u] = *reinterpret_cast<const float4*>(srow + (j < L ? j : 0));                               \
    }
    FP_LOAD_SEG(0);
    // thread 0 adds the previous segment's block sums (ascending) while the
    // current segment's exponentials are formed
    float Z = 0.0f;
    int zn = 0;
    for (int seg0 = 0; seg0 < L; seg0 += SEG) {
        if (seg0 + SEG - 1 <= pos) {
            // every key of the segment is causal and inside the sequence
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int jl = u * 1024 + 4 * tid;      // 4 consecutive keys, coalesced
                float4 v = buf[u];
                v.x = exp2_c(v.x - M, K);
                v.y = exp2_c(v.y - M, K);
                v.z = exp2_c(v.z - M, K);
                v.w = exp2_c(v.w - M, K);
                float* e = &es[jl / BS][jl % BS];
                e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
            }
        } else {
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int jl = u * 1024 + 4 * tid;
                const int j = seg0 + jl;
                float4 v = buf[u];
                const bool in = j < L;
                v.x = in && j <= pos ? exp2_c(v.x - M, K) : 0.0f;
                v.y = in && j + 1 <= pos ? exp2_c(v.y - M, K) : 0.0f;
                v.z = in && j + 2 <= pos ? exp2_c(v.z - M, K) : 0.0f;
                v.w = in && j + 3 <= pos ? exp2_c(v.w - M, K) : 0.0f;
                float* e = &es[jl / BS][jl % BS];
                e[0] = v.x; e[1] = v.y; e[2] = v.z; e[3] = v.w;
            }
        }
        if (tid == 0)
            for (int i = 0; i < zn; ++i) Z = Z + zs[i];
        __syncthreads();
        if (seg0 + SEG < L) { FP_LOAD_SEG(seg0 + SEG); }
        const int nbs = min(kRowSeg, (L - seg0 + BS - 1) / BS);
        if (tid < nbs) {
            float z = 0.0f;
            for (int jj = 0; jj < BS; jj += 16) {
                float v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = es[tid][jj + u];
#pragma unroll
                for (int u = 0; u < 16; ++u) z = z + v[u];
            }
            zs[tid] = z;
        }
        zn = nbs;
        __syncthreads();
    }
#undef FP_LOAD_SEG
    if (tid == 0) {
        for (int i = 0; i < zn; ++i) Z = Z + zs[i];
        rowmax[(size_t)bh * BS + row] = M;
        rowsum[(size_t)bh * BS + row] = Z;
        rz[(size_t)bh * BS + row] = 1.0f / Z;
    }
}

// ---------------------------------------------------------------------------
// K3b: line scores of the last block's probabilities p = exp2_c(s - M) * rz
// (0 for j > pos):
//   colsum[j]  = sum_i p[i][j],                        i ascending;
//   diagsum[o] = sum_{i: pos_i >= o} p[i][pos_i - o],  i ascending.
// Workgroup x owns columns j0 .. j0+W-1 and the offsets o = L - BS - j0 - t,
// t in [0, W): row i of such an offset reads column j0 + t + i, so one LDS
// tile of W + BS columns per row serves both sums (the BS extra columns are
// also in the next workgroup's tile: BS / W of the exponentials are formed
// twice).  W = 1024 where that still leaves at least 2048 workgroups, else
// 512 (measured: 0.48 -> 0.45 ms on the 128k layer, but 0.14 -> 0.16 ms on
// the 32k one, whose 1024 workgroups then fill the chip only once).  Rows
// are staged 8 at a time (at block 64 a chunk is not a whole number of
// float4 per thread: the last load covers only the first waves); every
// thread keeps its sums in registers across the chunks.  The tile holds p = e * rz (the
// product is rounded once whichever sum uses it).
// Once its columns are summed, a workgroup also forms the block sums
// t[kb] = sum of colsum over key block kb (j ascending) of the blocks its
// columns cover (W is a multiple of BS), into `blocksum`; the divergence
// kernel normalises them into the pooled true distribution.  The offsets
// above L - BS are summed by one more workgroup per head (x = ceil(L / W),
// line_tail below).  grid (ceil(L / W) + 1, BH).
// Rows that do not exist (L < BS) have M = rz = 0 and contribute zeros.
// ---------------------------------------------------------------------------
inline int line_width(int L, int BH) { return (long long)((L + 1023) / 1024) * BH >= 2048 ? 1024 : 512; }

// Offsets o = L - BS + 1 + t (t < BS - 1, o >= 0): only rows i > t reach
// them, at column i - t - 1.  Thread t sums offset t; the scattered scores
// are loaded eight at a time ahead of the (sequential, i ascending) sum.
template <int BS>
__device__ __forceinline__ void line_tail(const float* __restrict__ S, const float* sM, const float* sR,
                                          float* __restrict__ diag, int L, int NS, const Canon& K, int t) {
    const int o = L - BS + 1 + t;
    if (t >= BS - 1 || o < 0) return;
    float g = 0.0f;
    int i = t + 1;
    for (; i + 8 <= BS; i += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = S[(size_t)(i + u) * NS + (i + u - t - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float p = exp2_c(v[u] - sM[i + u], K) * sR[i + u];
            g = g + p;
        }
    }
    for (; i < BS; ++i) {
        const float p = exp2_c(S[(size_t)i * NS + (i - t - 1)] - sM[i], K) * sR[i];
        g = g + p;
    }
    diag[o] = g;
}

template <int BS, int W>
__global__ __launch_bounds__(256) void k_linesums(const float* __restrict__ s2, const float* __restrict__ rowmax,
                                                  const float* __restrict__ rz, float* __restrict__ colsum,
                                                  float* __restrict__ diagsum, float* __restrict__ blocksum,
                                                  int L, int NS, Canon K) {
    constexpr int RC = 8, TW = W + BS;
    static_assert(W % BS == 0 && RC * TW >= W, "block sums are staged in the row tile");
    __shared__ __attribute__((aligned(16))) float es[RC][TW];
    __shared__ float sM[BS], sR[BS];
    const int tid = threadIdx.x, bh = blockIdx.y;
    const int j0 = blockIdx.x * W;
    if (tid < BS) {
        sM[tid] = rowmax[(size_t)bh * BS + tid];
        sR[tid] = rz[(size_t)bh * BS + tid];
    }
    if (blockIdx.x == gridDim.x - 1) {
        // the diagonal tail of this head
        __syncthreads();
        if (tid < BS) line_tail<BS>(s2 + (size_t)bh * BS * NS, sM, sR, diagsum + (size_t)bh * L, L, NS, K, tid);
        return;
    }
    float cacc[W / 256], gacc[W / 256];
#pragma unroll
    for (int q = 0; q < W / 256; ++q) cacc[q] = gacc[q] = 0.0f;
    const float* S = s2 + (size_t)bh * BS * NS;
    // Each thread loads NL float4 of a chunk; the next chunk's loads are in
    // flight while the current one is summed.  Columns at or past L read
    // column 0 of their row and count as 0.
    constexpr int N4 = RC * TW / 4;                 // float4 per chunk
    constexpr int NL = (N4 + 255) / 256;
    static_assert(N4 * 4 == RC * TW && (N4 % 256) % 64 == 0, "chunk tiling: whole waves per load");
    float4 buf[NL];
    // the last load of a chunk may cover only its first waves (wave-uniform)
#define FP_IN_CHUNK(n_) (N4 % 256 == 0 || (n_) < NL - 1 || tid < N4 % 256)
#define FP_LOAD_CHUNK(i0_)                                                                                 \
    _Pragma("unroll") for (int n = 0; n < NL; ++n) {                                                     \
        const int e4 = tid + 256 * n;                                                                    \
        if (!FP_IN_CHUNK(n)) continue;                                                                   \
        const int ii = e4 / (TW / 4), cc = 4 * (e4 % (TW / 4));                                          \
        const int j = j0 + cc;                                                                           \
        buf[n] = *reinterpret_cast<const float4*>(S + (size_t)((i0_) + ii) * NS + (j < L ? j : 0));       \
    }
    FP_LOAD_CHUNK(0);
    __syncthreads();
    for (int i0 = 0; i0 < BS; i0 += RC) {
        if (j0 + TW - 1 <= L - BS) {
            // every column of the tile is causal for every row and inside the sequence
#pragma unroll
            for (int n = 0; n < NL; ++n) {
                const int e4 = tid + 256 * n;
                if (!FP_IN_CHUNK(n)) continue;
                const int ii = e4 / (TW / 4), cc = 4 * (e4 % (TW / 4));
                const int i = i0 + ii;
                const float4 v = buf[n];
                const float M = sM[i], r = sR[i];
                float4 x;
                x.x = exp2_c(v.x - M, K) * r;
                x.y = exp2_c(v.y - M, K) * r;
                x.z = exp2_c(v.z - M, K) * r;
                x.w = exp2_c(v.w - M, K) * r;
                *reinterpret_cast<float4*>(&es[ii][cc]) = x;
            }
        } else {
#pragma unroll
            for (int n = 0; n < NL; ++n) {
                const int e4 = tid + 256 * n;
                if (!FP_IN_CHUNK(n)) continue;
                const int ii = e4 / (TW / 4), cc = 4 * (e4 % (TW / 4));
                const int i = i0 + ii, j = j0 + cc, pos = L - BS + i;
                const float4 v = buf[n];
                const float M = sM[i], r = sR[i];
                const bool in = j < L;
                float4 x;
                x.x = in && j <= pos ? exp2_c(v.x - M, K) * r : 0.0f;
                x.y = in && j + 1 <= pos ? exp2_c(v.y - M, K) * r : 0.0f;
                x.z = in && j + 2 <= pos ? exp2_c(v.z - M, K) * r : 0.0f;
                x.w = in && j + 3 <= pos ? exp2_c(v.w - M, K) * r : 0.0f;
                *reinterpret_cast<float4*>(&es[ii][cc]) = x;
            }
        }
        __syncthreads();
        if (i0 + RC < BS) { FP_LOAD_CHUNK(i0 + RC); }
#pragma unroll 4
        for (int ii = 0; ii < RC; ++ii) {
            const int i = i0 + ii;
#pragma unroll
            for (int q = 0; q < W / 256; ++q) {
                const int t = tid + 256 * q;
                cacc[q] = cacc[q] + es[ii][t];
                gacc[q] = gacc[q] + es[ii][t + i];
            }
        }
        __syncthreads();
    }
#undef FP_LOAD_CHUNK
#undef FP_IN_CHUNK
    float* cs = &es[0][0];      // free after the last chunk's barrier
#pragma unroll
    for (int q = 0; q < W / 256; ++q) {
        const int t = tid + 256 * q;
        const int j = j0 + t;
        if (j < L) colsum[(size_t)bh * L + j] = cacc[q];
        const int o = L - BS - j0 - t;
        if (o >= 0) diagsum[(size_t)bh * L + o] = gacc[q];
        cs[t] = cacc[q];
    }
    __syncthreads();
    // block sums of the covered blocks, sequential over j ascending; the
    // values read ahead 16 at a time
    if (tid < W / BS) {
        const int nb = (L + BS - 1) / BS, kb = j0 / BS + tid;
        if (kb < nb) {
            const int n = min(BS, L - kb * BS);
            const float* c = cs + tid * BS;
            float t = 0.0f;
            int jj = 0;
            for (; jj + 16 <= n; jj += 16) {
                float v[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) v[u] = c[jj + u];
#pragma unroll
                for (int u = 0; u < 16; ++u) t = t + v[u];
            }
            for (; jj < n; ++jj) t = t + c[jj];
            blocksum[(size_t)bh * nb + kb] = t;
        }
    }
}

// ---------------------------------------------------------------------------
// K4: estimated block map  A[qb][kb] = softmax_{kb <= qb}(fp32(qbar_qb . kbar_kb) * C)
// (products and sums rounded separately, t ascending; row max subtracted,
// exp2_c, sum over kb ascending, rounded division).  Stored as the causal
// triangle, row-major.  A workgroup handles R consecutive query-block rows,
// so every pooled key row it reads serves R dot products.
// grid (ceil(nb / R), BH), dynamic LDS R * nb floats.
// ---------------------------------------------------------------------------
template <int R, int D>
__global__ __launch_bounds__(256) void k_estimate(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                  float* __restrict__ ahat, int nb, int Hq, int Hkv,
                                                  int group, Canon K) {
    extern __shared__ float sc[];              // [R][nb]
    __shared__ __attribute__((aligned(16))) float qs[R][D];
    __shared__ float red[R][256];
    __shared__ float Mr[R], Zr[R];
    const int tid = threadIdx.x, bh = blockIdx.y;
    const int q0 = blockIdx.x * R;
    const int b = bh / Hq, h = bh % Hq;
    const size_t kvbh = (size_t)b * Hkv + h / group;
    for (int e = tid; e < R * D; e += 256) {
        const int r = e / D, t = e % D;
        qs[r][t] = (q0 + r < nb) ? qbar[((size_t)bh * nb + q0 + r) * D + t] : 0.0f;
    }
    __syncthreads();
    const int qlast = min(q0 + R - 1, nb - 1);
    float mx[R];
#pragma unroll
    for (int r = 0; r < R; ++r) mx[r] = -INFINITY;
    for (int kb = tid; kb <= qlast; kb += 256) {
        const float4* kr = reinterpret_cast<const float4*>(kbar + (kvbh * nb + kb) * D);
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll 4
        for (int c = 0; c < D / 4; ++c) {
            const float4 v = kr[c];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float4 qv = *reinterpret_cast<const float4*>(&qs[r][4 * c]);
                float p;
                p = qv.x * v.x; acc[r] = acc[r] + p;
                p = qv.y * v.y; acc[r] = acc[r] + p;
                p = qv.z * v.z; acc[r] = acc[r] + p;
                p = qv.w * v.w; acc[r] = acc[r] + p;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (kb <= q0 + r) {
                const float s = acc[r] * K.C;
                sc[r * nb + kb] = s;
                mx[r] = fmaxf(mx[r], s);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) red[r][tid] = mx[r];
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s)
#pragma unroll
            for (int r = 0; r < R; ++r) red[r][tid] = fmaxf(red[r][tid], red[r][tid + s]);
        __syncthreads();
    }
    if (tid < R) Mr[tid] = red[tid][0];
    __syncthreads();
    for (int kb = tid; kb <= qlast; kb += 256)
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (kb <= q0 + r) sc[r * nb + kb] = exp2_c(sc[r * nb + kb] - Mr[r], K);
    __syncthreads();
    if (tid < R && q0 + tid < nb) {
        // sequential sum; the LDS reads go out 16 at a time ahead of the adds
        const float* zr = sc + tid * nb;
        const int n = q0 + tid + 1;
        float Z = 0.0f;
        int kb = 0;
        for (; kb + 16 <= n; kb += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = zr[kb + u];
#pragma unroll
            for (int u = 0; u < 16; ++u) Z = Z + v[u];
        }
        for (; kb < n; ++kb) Z = Z + zr[kb];
        Zr[tid] = Z;
    }
    __syncthreads();
    const long long tri = (long long)nb * (nb + 1) / 2;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int qb = q0 + r;
        if (qb >= nb) break;
        float* out = ahat + (size_t)bh * tri + (size_t)qb * (qb + 1) / 2;
        for (int kb = tid; kb <= qb; kb += 256) out[kb] = sc[r * nb + kb] / Zr[r];
    }
}

// ---------------------------------------------------------------------------
// K5: block-pooled true distribution and pattern determination.
// a_true[kb] = t[kb] / T with t the block sums of colsum (formed by the line
// kernel) and T = sum of t over kb ascending, in fp32 (written back over t).
// P = last row of the estimate, Q = a_true;
// JSD = 0.5 * sum_kb (P ln(P/m) + Q ln(Q/m)), m = (P + Q)/2, terms with a zero
// probability dropped, sum ascending in binary64; D = sqrt(JSD);
// query-aware iff D < tau.  One workgroup per head.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_jsd(const float* __restrict__ ahat, float* __restrict__ atrue,
                                             double* __restrict__ djs, unsigned char* __restrict__ pattern,
                                             int nb, double tau, Canon K) {
    __shared__ double terms[kMaxBlocks];
    __shared__ float ts[kMaxBlocks];
    __shared__ float Tsh;
    const int tid = threadIdx.x, bh = blockIdx.x;
    float* at = atrue + (size_t)bh * nb;
    for (int kb = tid; kb < nb; kb += 256) ts[kb] = at[kb];
    __syncthreads();
    if (tid == 0) {
        float T = 0.0f;
        int kb = 0;
        for (; kb + 16 <= nb; kb += 16) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = ts[kb + u];
#pragma unroll
            for (int u = 0; u < 16; ++u) T = T + v[u];
        }
        for (; kb < nb; ++kb) T = T + ts[kb];
        Tsh = T;
    }
    __syncthreads();
    const long long tri = (long long)nb * (nb + 1) / 2;
    const float* last = ahat + (size_t)bh * tri + (size_t)(nb - 1) * nb / 2;
    for (int kb = tid; kb < nb; kb += 256) {
        const float a = ts[kb] / Tsh;
        at[kb] = a;
        const double P = (double)last[kb];
        const double Q = (double)a;
        const double m = 0.5 * (P + Q);
        double tP = 0.0, tQ = 0.0;
        if (P > 0.0) tP = P * ln_c(P / m, K);
        if (Q > 0.0) tQ = Q * ln_c(Q / m, K);
        terms[kb] = tP + tQ;
    }
    __syncthreads();
    if (tid == 0) {
        double acc = 0.0;
        for (int kb = 0; kb < nb; ++kb) acc = acc + terms[kb];
        const double jsd = 0.5 * acc;
        const double D = sqrt(jsd > 0.0 ? jsd : 0.0);
        djs[bh] = D;
        pattern[bh] = (D < tau) ? 1 : 0;
    }
}

// ---------------------------------------------------------------------------
// K6: cumulative-attention selection, exact.  For every list (per head: the
// flattened estimate for query-aware heads; column sums and diagonal sums
// for vertical-slash heads) find K* = the key of the last element of the
// shortest prefix, in (value desc, index asc) order, whose fixed-point mass
// reaches T = ceil(G U / 2^24).  Radix selection from the most significant
// key bits, 11 bits per pass, with mass (not count) histograms.
// ---------------------------------------------------------------------------
struct ListRef {
    const float* x;
    long long len;
};

__device__ __forceinline__ ListRef list_of(const PlanDev& P, int list) {
    const int bh = list >> 1, slot = list & 1;
    ListRef r{nullptr, 0};
    if (P.pattern[bh] == kPatternQueryAware) {
        // the query-wise variant selects row by row in k_lists instead
        if (slot == 0 && !P.qa_querywise) { r.x = P.ahat + (size_t)bh * P.tri; r.len = P.tri; }
    } else {
        r.x = (slot == 0 ? P.colsum : P.diagsum) + (size_t)bh * P.L;
        r.len = P.L;
    }
    return r;
}

// Clears the lists' states (their totals are summed into them) and the
// histogram buffer of the first pass.
__global__ __launch_bounds__(256) void k_sel_reset(SelState* __restrict__ st, unsigned long long* __restrict__ hist,
                                                   int nlists) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < nlists) {
        SelState s = {};
        st[i] = s;
    }
    const long long n = (long long)nlists * kRadixBins;
    for (long long t = i; t < n; t += (long long)gridDim.x * 256) hist[t] = 0ull;
}

__global__ __launch_bounds__(256) void k_sel_total(PlanDev P, SelState* __restrict__ st, int chunk) {
    __shared__ unsigned long long red[256];
    const int list = blockIdx.y, tid = threadIdx.x;
    const ListRef L = list_of(P, list);
    const long long base = (long long)blockIdx.x * chunk;
    unsigned long long s = 0;
    if (base < L.len) {
        const long long end = min(base + (long long)chunk, L.len);
        for (long long i = base + tid; i < end; i += 256) s += fixed_u(L.x[i]);
    }
    red[tid] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    if (tid == 0 && red[0]) atomicAdd(&st[list].U, red[0]);
}

// State of a list before its first pass, from its total fixed-point mass U.
__device__ __forceinline__ SelState sel_first_state(unsigned long long U, long long len, unsigned long long G) {
    SelState s = {};
    const unsigned long long hi = U >> kGammaShift, lo = U & ((1ull << kGammaShift) - 1);
    const unsigned long long T = G * hi + ((G * lo + ((1ull << kGammaShift) - 1)) >> kGammaShift);
    s.U = U;
    s.T = T;
    s.R = T;
    s.prefix = 0;
    s.ibits = index_bits(len > 0 ? len : 1);
    s.pos = 31 + s.ibits;
    s.active = (len > 0 && T > 0) ? 1 : 0;
    s.has = s.active;
    s.kstar = 0;
    return s;
}

// Resolves the next digit of a list's threshold key from the mass histogram
// `gh` of the pass that read it: the lowest digit at which the mass of all
// lower digits plus its own reaches the remaining target R.  Called by all
// 256 threads of a workgroup with the same state; every thread gets the
// same result.  Inactive lists come back unchanged.
__device__ SelState sel_advance(const SelState s, const unsigned long long* __restrict__ gh) {
    constexpr int PER = kRadixBins / 256;
    __shared__ unsigned long long wsum[4];
    __shared__ int found;
    __shared__ SelState res;
    if (!s.active) return s;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    unsigned long long v[PER];
    unsigned long long run = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        v[r] = gh[tid * PER + r];
        run += v[r];
    }
    // inclusive prefix of the per-thread totals: within each wave by
    // shuffles, then across the four waves
    unsigned long long x = run;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_up(x, (unsigned)o, 64);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    if (tid == 0) {
        found = kRadixBins;
        res = s;
    }
    __syncthreads();
    unsigned long long cum = x - run;    // mass of all lower digits
    for (int w2 = 0; w2 < wid; ++w2) cum += wsum[w2];
    const int w = s.pos < kRadixBits ? s.pos : kRadixBits;
    int mine = kRadixBins;
    unsigned long long below = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int dgt = tid * PER + r;
        if (mine == kRadixBins && dgt < (1 << w) && cum + v[r] >= s.R) {
            mine = dgt;
            below = cum;
        }
        cum += v[r];
    }
    if (mine < kRadixBins) atomicMin(&found, mine);
    __syncthreads();
    if (mine == found && mine < kRadixBins) {
        SelState t = s;
        t.R -= below;
        t.prefix = (t.prefix << w) | (unsigned long long)mine;
        t.pos -= w;
        if (t.pos == 0) {
            t.active = 0;
            t.kstar = t.prefix;
        }
        res = t;
    }
    __syncthreads();
    return res;
}

// Radix pass k of every list: the state before the pass (pass 0: from the
// list's total; later passes: the previous state advanced by the previous
// pass's histogram, by every workgroup of the list alike; workgroup 0
// stores it), then the mass histogram of the next digit over the elements
// whose key matches the resolved prefix.  The histograms rotate through
// kSelHistBufs buffers: pass k reads buffer k - 1, fills buffer k and (its
// workgroup 0) clears buffer k + 1, which pass k - 1 was the last to read and
// pass k + 1 fills.  grid (chunks of `chunk` elements, lists).
__global__ __launch_bounds__(256) void k_sel_pass(PlanDev P, int k, int nlists, unsigned long long G, int chunk) {
    __shared__ unsigned long long hist[kRadixBins];
    const int list = blockIdx.y, tid = threadIdx.x;
    const ListRef L = list_of(P, list);
    const long long base = (long long)blockIdx.x * chunk;
    // workgroups past the list's end have nothing to count (workgroup 0
    // still stores the state)
    if (blockIdx.x > 0 && base >= L.len) return;
    const SelState s = k == 0 ? sel_first_state(P.sel[list].U, L.len, G)
                              : sel_advance(P.selk[(size_t)(k - 1) * nlists + list],
                                            P.hist + ((size_t)((k - 1) % kSelHistBufs) * nlists + list) * kRadixBins);
    if (blockIdx.x == 0) {
        if (tid == 0) P.selk[(size_t)k * nlists + list] = s;
        unsigned long long* nx = P.hist + ((size_t)((k + 1) % kSelHistBufs) * nlists + list) * kRadixBins;
        for (int i = tid; i < kRadixBins; i += 256) nx[i] = 0ull;
    }
    if (!s.active || base >= L.len) return;
    for (int i = tid; i < kRadixBins; i += 256) hist[i] = 0ull;
    __syncthreads();
    const int w = s.pos < kRadixBits ? s.pos : kRadixBits;
    const int shift = s.pos - w;
    const unsigned long long dmask = (1ull << w) - 1ull;
    const long long end = min(base + (long long)chunk, L.len);
    for (long long i = base + tid; i < end; i += 256) {
        const float x = L.x[i];
        const unsigned long long key = order_key(x, i, s.ibits);
        if ((key >> s.pos) == s.prefix) {
            const unsigned long long u = fixed_u(x);
            if (u) atomicAdd(&hist[(key >> shift) & dmask], u);
        }
    }
    __syncthreads();
    unsigned long long* gh = P.hist + ((size_t)(k % kSelHistBufs) * nlists + list) * kRadixBins;
    for (int i = tid; i < kRadixBins; i += 256)
        if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// The final state of every list: the state before the last pass advanced
// by its histogram.  One workgroup per list.
__global__ __launch_bounds__(256) void k_sel_final(PlanDev P, int passes, int nlists) {
    const int list = blockIdx.x;
    const SelState s = sel_advance(P.selk[(size_t)(passes - 1) * nlists + list],
                                   P.hist + ((size_t)((passes - 1) % kSelHistBufs) * nlists + list) * kRadixBins);
    if (threadIdx.x == 0) P.sel[list] = s;
}

// ---------------------------------------------------------------------------
// K7a: vertical-slash lines -> block flags (any-touch rule).
// colblk[kb]: some selected column j in key block kb.
// diagA[a]:   some selected offset o with o / BS == a;
// diagB[a]:   some selected offset o with o / BS == a and o % BS > 0.
// diagT[a]:   some selected offset o with o / BS == a and o % BS < tail
//             (tail = query rows of the last, possibly partial, block row).
// Block (qb, kb) is touched iff colblk[kb] or diagA[qb-kb] (diagT[qb-kb] in
// the last block row) or diagB[qb-kb-1].  grid (nb, BH), BS threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void k_vs_flags(PlanDev P, const SelState* __restrict__ st) {
    __shared__ int f[5];
    __shared__ unsigned char selc_s[kMaxBlock], selg_s[kMaxBlock];
    const int kb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    if (P.mode_all || P.pattern[bh] == kPatternQueryAware) return;
    if (tid < 5) f[tid] = 0;
    __syncthreads();
    const SelState sc = st[2 * bh], sg = st[2 * bh + 1];
    const long long j = (long long)kb * P.BS + tid;
    const bool in = j < P.L;
    const float xc = in ? P.colsum[(size_t)bh * P.L + j] : 0.0f;
    const float xg = in ? P.diagsum[(size_t)bh * P.L + j] : 0.0f;
    const bool selc = in && sc.has && order_key(xc, j, sc.ibits) <= sc.kstar;
    const bool selg = in && sg.has && order_key(xg, j, sg.ibits) <= sg.kstar;
    if (selc) f[0] = 1;
    if (selg) f[1] = 1;
    if (selg && tid > 0) f[2] = 1;
    if (selg && tid < P.tail) f[3] = 1;
    if (selc && P.vs_token) atomicAdd(&f[4], 1);
    selc_s[tid] = selc;
    selg_s[tid] = selg;
    __syncthreads();
    if (tid == 0) {
        const size_t o = (size_t)bh * P.nb + kb;
        P.colblk[o] = (unsigned char)f[0];
        P.diagA[o] = (unsigned char)f[1];
        P.diagB[o] = (unsigned char)f[2];
        P.diagT[o] = (unsigned char)f[3];
        if (P.vs_token) P.colcount[o] = f[4];
    }
    if (P.cap_blocks > 0 && tid == 0) {
        // line mass for the per-row cap, float32 sums in ascending index:
        // colmass[kb] = selected c[j] of this key block; diagmass[kb] starts
        // with the selected g[o] of offsets in block kb (the terms with
        // o % BS > 0 of block kb - 1 are added by k_diag_mass afterwards)
        const float* cs = P.colsum + (size_t)bh * P.L + (size_t)kb * P.BS;
        const float* gs = P.diagsum + (size_t)bh * P.L + (size_t)kb * P.BS;
        float cm = 0.0f, dm = 0.0f;
        for (int r = 0; r < P.BS; ++r) {
            if (selc_s[r]) cm = cm + cs[r];
            if (selg_s[r]) dm = dm + gs[r];
        }
        P.colmass[(size_t)bh * P.nb + kb] = cm;
        P.diagmass[(size_t)bh * P.nb + kb] = dm;
    }
}

// Second half of diagmass[a]: the selected offsets o of block a - 1 with
// o % BS > 0, ascending, added after the first half.  grid (nb, BH).
__global__ __launch_bounds__(64) void k_diag_mass(PlanDev P, const SelState* __restrict__ st) {
    const int a = blockIdx.x, bh = blockIdx.y;
    if (threadIdx.x != 0 || a == 0 || P.mode_all || P.pattern[bh] == kPatternQueryAware) return;
    const SelState sg = st[2 * bh + 1];
    const long long base = (long long)(a - 1) * P.BS;
    const float* gs = P.diagsum + (size_t)bh * P.L;
    float dm = P.diagmass[(size_t)bh * P.nb + a];
    for (int r = 1; r < P.BS && base + r < P.L; ++r) {
        const float x = gs[base + r];
        if (sg.has && order_key(x, base + r, sg.ibits) <= sg.kstar) dm = dm + x;
    }
    P.diagmass[(size_t)bh * P.nb + a] = dm;
}

// ---------------------------------------------------------------------------
// Token-granular columns: colptr[kb] = selected columns in key blocks < kb
// (exclusive prefix over the head's blocks, colptr[nb] = all of them), then
// colidx[colptr[kb] + rank] = the block's selected columns in ascending order.
// Heads without token columns (query-aware, gamma = 1) get colptr = 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_col_scan(PlanDev P) {
    constexpr int PER = kMaxBlocks / 256;
    __shared__ int tot[256];
    const int bh = blockIdx.x, tid = threadIdx.x, nb = P.nb;
    const bool vs = !P.mode_all && P.pattern[bh] != kPatternQueryAware;
    int v[PER];
    int run = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int kb = tid * PER + r;
        v[r] = (vs && kb < nb) ? P.colcount[(size_t)bh * nb + kb] : 0;
        run += v[r];
    }
    tot[tid] = run;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
        const int add = tid >= o ? tot[tid - o] : 0;
        __syncthreads();
        tot[tid] += add;
        __syncthreads();
    }
    int cum = tot[tid] - run;
    int* cp = P.colptr + (size_t)bh * (nb + 1);
#pragma unroll
    for (int r = 0; r < PER; ++r) {
        const int kb = tid * PER + r;
        if (kb < nb) cp[kb] = cum;
        cum += v[r];
    }
    if (tid == 255) cp[nb] = tot[255];
}

__global__ __launch_bounds__(128) void k_col_compact(PlanDev P, const SelState* __restrict__ st) {
    __shared__ int wcount[2];
    const int kb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (P.mode_all || P.pattern[bh] == kPatternQueryAware) return;
    const SelState sc = st[2 * bh];
    const long long j = (long long)kb * P.BS + tid;
    const bool in = j < P.L;
    const float xc = in ? P.colsum[(size_t)bh * P.L + j] : 0.0f;
    const bool selc = in && sc.has && order_key(xc, j, sc.ibits) <= sc.kstar;
    const unsigned long long bal = __ballot(selc);
    if (lane == 0) wcount[w] = __popcll(bal);
    __syncthreads();
    const int rank = (w == 1 ? wcount[0] : 0) + __popcll(bal & ((1ull << lane) - 1ull));
    if (selc) P.colidx[(size_t)bh * P.L + P.colptr[(size_t)bh * (P.nb + 1) + kb] + rank] = (int)j;
}

// ---------------------------------------------------------------------------
// K7b: per (head, query-block row) block list: selected blocks, topped up to
// the minimum budget with unselected blocks nearest the diagonal first, in
// ascending key-block order at lists[bh][row (row+1)/2 + ...].
// One wave per row, 4 rows per workgroup.
// ---------------------------------------------------------------------------
// Row-selection keys: value descending, then key block ascending.
constexpr int kRowIdxBits = 12;

__device__ __forceinline__ bool member(const PlanDev& P, const SelState& s0, int bh, int qb, int kb, bool qa,
                                       const float* arow, long long toff, bool rhas, unsigned long long rkey) {
    if (P.mode_all) return true;
    if (qa && P.qa_querywise) return rhas && order_key(arow[kb], kb, kRowIdxBits) <= rkey;
    if (qa) return s0.has && order_key(arow[kb], toff + kb, s0.ibits) <= s0.kstar;
    const size_t base = (size_t)bh * P.nb;
    const int a = qb - kb;
    const unsigned char* own = qb == P.nb - 1 ? P.diagT : P.diagA;
    return (!P.vs_token && P.colblk[base + kb]) || own[base + a] || (a >= 1 && P.diagB[base + a - 1]);
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
    for (int o = 32; o >= 1; o >>= 1) { const unsigned long long w = __shfl_xor(v, o); v = w < v ? w : v; }
    return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
    for (int o = 32; o >= 1; o >>= 1) { const unsigned long long w = __shfl_xor(v, o); v = w > v ? w : v; }
    return v;
}

// Query-wise selection of one estimated row a[0..len) by one wave: the
// smallest key K with mass(keys <= K) >= T, T = ceil(G U / 2^24) of the
// row's own fixed-point total U, found bit by bit from the highest bit in
// which the row's keys differ.  Returns false when T = 0 (nothing selected).
__device__ bool row_select(const float* a, int len, unsigned long long G, unsigned long long* kout) {
    const int lane = threadIdx.x & 63;
    unsigned long long U = 0ull, kmin = ~0ull, kmax = 0ull;
    for (int kb = lane; kb < len; kb += 64) {
        const float x = a[kb];
        U += fixed_u(x);
        const unsigned long long key = order_key(x, kb, kRowIdxBits);
        kmin = key < kmin ? key : kmin;
        kmax = key > kmax ? key : kmax;
    }
    U = wave_sum_u64(U);
    kmin = wave_min_u64(kmin);
    kmax = wave_max_u64(kmax);
    const unsigned long long hi = U >> kGammaShift, lo = U & ((1ull << kGammaShift) - 1);
    const unsigned long long T = G * hi + ((G * lo + ((1ull << kGammaShift) - 1)) >> kGammaShift);
    if (T == 0ull) return false;
    const unsigned long long diff = kmin ^ kmax;
    if (diff == 0ull) {
        *kout = kmin;
        return true;
    }
    const int top = 63 - __clzll((long long)diff);
    unsigned long long prefix = kmin & ~((2ull << top) - 1ull);
    unsigned long long below = 0ull;    // mass of the keys below the current range
    for (int b = top; b >= 0; --b) {
        unsigned long long m0 = 0ull;
        for (int kb = lane; kb < len; kb += 64) {
            const float x = a[kb];
            const unsigned long long key = order_key(x, kb, kRowIdxBits);
            if ((key >> (b + 1)) == (prefix >> (b + 1)) && !((key >> b) & 1ull)) m0 += fixed_u(x);
        }
        m0 = wave_sum_u64(m0);
        if (below + m0 < T) {
            below += m0;
            prefix |= 1ull << b;
        }
    }
    *kout = prefix;
    return true;
}

// Score of block kb in row qb for the maximum-budget cap (>= 0).
__device__ __forceinline__ float cap_score(const PlanDev& P, int bh, int qb, int kb, bool qa, const float* arow) {
    if (qa || P.mode_all) return arow[kb];
    const size_t base = (size_t)bh * P.nb;
    return P.colmass[base + kb] + P.diagmass[base + (qb - kb)];
}

// Cap order: score descending, then key block descending (nearest the diagonal).
__device__ __forceinline__ unsigned long long cap_key(float score, int kb) {
    return ((unsigned long long)(0x7FFFFFFFu - __float_as_uint(score)) << 12) | (unsigned long long)(4095 - kb);
}

__global__ __launch_bounds__(256) void k_lists(PlanDev P, const SelState* __restrict__ st) {
    // membership of each 64-block chunk of the row, one ballot per chunk
    __shared__ unsigned long long masks[4][kMaxBlocks / 64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int bh = blockIdx.y, qb = blockIdx.x * 4 + wv;
    if (qb >= P.nb) return;
    const bool qa = P.pattern[bh] == kPatternQueryAware;
    const SelState s0 = st[2 * bh];
    const long long toff = (long long)qb * (qb + 1) / 2;
    const float* arow = P.ahat + (size_t)bh * P.tri + toff;
    const int nch = qb / 64 + 1;
    unsigned long long* mk = masks[wv];
    unsigned long long rkey = 0ull;
    const bool rhas = qa && P.qa_querywise && !P.mode_all && row_select(arow, qb + 1, P.G, &rkey);
    int cnt = 0;
    for (int ch = 0; ch < nch; ++ch) {
        const int kb = 64 * ch + lane;
        const unsigned long long bal =
            __ballot(kb <= qb && member(P, s0, bh, qb, kb, qa, arow, toff, rhas, rkey));
        if (lane == 0) mk[ch] = bal;
        cnt += __popcll(bal);
    }
    __builtin_amdgcn_wave_barrier();
    // minimum budget: the `need` unselected blocks nearest the diagonal, i.e.
    // every unselected kb >= cut
    const int want = min(qb + 1, P.floor_blocks);
    int need = want - cnt;
    int cut = qb + 1;
    for (int ch = nch - 1; need > 0 && ch >= 0; --ch) {
        const int valid = min(64, qb + 1 - 64 * ch);
        const unsigned long long vmask = valid == 64 ? ~0ull : ((1ull << valid) - 1ull);
        unsigned long long un = ~mk[ch] & vmask;
        const int c = __popcll(un);
        if (need <= c) {
            for (int t = 1; t < need; ++t) un &= ~(1ull << (63 - __clzll((long long)un)));
            cut = 64 * ch + (63 - __clzll((long long)un));
            need = 0;
        } else {
            need -= c;
        }
    }
    // final membership: selected, or filled for the minimum budget
    int total = 0;
    for (int ch = 0; ch < nch; ++ch) {
        const int valid = min(64, qb + 1 - 64 * ch);
        const unsigned long long vmask = valid == 64 ? ~0ull : ((1ull << valid) - 1ull);
        unsigned long long fill = 0ull;
        if (cut <= 64 * ch + 63) fill = cut <= 64 * ch ? ~0ull : ~((1ull << (cut - 64 * ch)) - 1ull);
        const unsigned long long m = (mk[ch] | fill) & vmask;
        if (lane == 0) mk[ch] = m;
        total += __popcll(m);
    }
    __builtin_amdgcn_wave_barrier();
    // maximum budget: keep the cap_blocks members with the smallest cap keys
    if (P.cap_blocks > 0 && total > P.cap_blocks) {
        unsigned long long prefix = 0ull;
        int rem = P.cap_blocks;
        for (int b = 42; b >= 0; --b) {
            int c0 = 0;
            for (int ch = 0; ch < nch; ++ch) {
                const int kb = 64 * ch + lane;
                bool in = false;
                if ((mk[ch] >> lane) & 1ull) {
                    const unsigned long long key = cap_key(cap_score(P, bh, qb, kb, qa, arow), kb);
                    in = (key >> (b + 1)) == (prefix >> (b + 1)) && !((key >> b) & 1ull);
                }
                c0 += __popcll(__ballot(in));
            }
            if (rem > c0) {
                rem -= c0;
                prefix |= 1ull << b;
            }
        }
        // prefix is now the key of the cap_blocks-th kept block
        total = 0;
        for (int ch = 0; ch < nch; ++ch) {
            const int kb = 64 * ch + lane;
            bool keep = false;
            if ((mk[ch] >> lane) & 1ull) keep = cap_key(cap_score(P, bh, qb, kb, qa, arow), kb) <= prefix;
            const unsigned long long m = __ballot(keep);
            if (lane == 0) mk[ch] = m;
            total += __popcll(m);
        }
        __builtin_amdgcn_wave_barrier();
    }
    int* out = P.lists + (size_t)bh * P.tri + toff;
    int written = 0;
    for (int ch = 0; ch < nch; ++ch) {
        const int kb = 64 * ch + lane;
        const unsigned long long m = mk[ch];
        const bool f = (m >> lane) & 1ull;
        if (f) out[written + __popcll(m & ((1ull << lane) - 1ull))] = kb;
        written += __popcll(m);
    }
    if (lane == 0) P.counts[(size_t)bh * P.nb + qb] = written;
}

// Per-head block totals from the rows' counts, one workgroup per head (a
// per-row atomic add into one counter per head serialised about 1000 adds
// on each address).
__global__ __launch_bounds__(256) void k_head_totals(const int* __restrict__ counts,
                                                     unsigned long long* __restrict__ tot, int nb) {
    __shared__ unsigned long long red[256];
    const int bh = blockIdx.x, tid = threadIdx.x;
    unsigned long long s = 0ull;
    for (int r = tid; r < nb; r += 256) s += (unsigned long long)counts[(size_t)bh * nb + r];
    red[tid] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] += red[tid + o];
        __syncthreads();
    }
    if (tid == 0) tot[bh] = red[0];
}

__global__ __launch_bounds__(256) void k_fill_u32(unsigned int* __restrict__ p, unsigned int v, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = v;
}

// Small host tables (the attention segment table) copied to the device by
// value through kernel arguments, 2 KB per launch: a copy from pageable host
// memory may be serialized with the host by the runtime.
struct UploadChunk {
    unsigned int w[512];
};
__global__ __launch_bounds__(256) void k_upload(unsigned int* __restrict__ dst, UploadChunk c, int n) {
    for (int i = threadIdx.x; i < n; i += 256) dst[i] = c.w[i];
}

// Three buffers zeroed by one launch (blockIdx.y picks the buffer).
__global__ __launch_bounds__(256) void k_zero3_u32(unsigned int* __restrict__ a, long long na,
                                                   unsigned int* __restrict__ b, long long nb,
                                                   unsigned int* __restrict__ c, long long nc) {
    unsigned int* p = blockIdx.y == 0 ? a : blockIdx.y == 1 ? b : c;
    const long long n = blockIdx.y == 0 ? na : blockIdx.y == 1 ? nb : nc;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = 0u;
}

// probes of the canonical functions
__global__ __launch_bounds__(256) void k_probe_exp2(const float* x, float* y, long long n, Canon K) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = exp2_c(x[i], K);
}
__global__ __launch_bounds__(256) void k_probe_ln(const double* x, double* y, long long n, Canon K) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = ln_c(x[i], K);
}
__global__ __launch_bounds__(256) void k_probe_sqrt(const double* x, double* y, long long n) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) y[i] = sqrt(x[i]);
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
static inline unsigned grid1(long long n, int per = 256) { return (unsigned)((n + per - 1) / per); }

template <int D>
static hipError_t launch_plan_t(const PlanArgs& a, PlanDev& P, hipStream_t st) {
    const int BS = P.BS, nb = P.nb, L = P.L, NS = P.NS, BH = P.BH;
    const int bkv = a.nseq * a.Hkv;
    const int group = a.Hq / a.Hkv;
    // K1 (pooling reads Q and K from HBM) and K4 (the estimated map from the
    // pooled vectors) run on the auxiliary stream, when there is one, next to
    // the VALU-bound score kernels; K5 joins them.
    hipStream_t ps = st;
    hipEvent_t fork = nullptr, join = nullptr;
    hipError_t he = hipSuccess;
    if (a.aux) {
        he = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
        if (he == hipSuccess) he = hipEventCreateWithFlags(&join, hipEventDisableTiming);
        if (he == hipSuccess) he = hipEventRecord(fork, st);
        if (he == hipSuccess) he = hipStreamWaitEvent(a.aux, fork, 0);
        if (he != hipSuccess) {
            if (fork) (void)hipEventDestroy(fork);
            if (join) (void)hipEventDestroy(join);
            return he;
        }
        ps = a.aux;
    }
    const unsigned pg = (unsigned)((nb + 256 / (D / 8) - 1) / (256 / (D / 8)));
    if (a.dtype_bf16) {
        hipLaunchKernelGGL((k_pool<bf16_t, D>), dim3(pg, BH), dim3(256), 0, ps, (const bf16_t*)a.q, a.qs, a.Hq, P.qbar, L, BS);
        hipLaunchKernelGGL((k_pool<bf16_t, D>), dim3(pg, bkv), dim3(256), 0, ps, (const bf16_t*)a.k, a.ks, a.Hkv, P.kbar, L, BS);
    } else {
        hipLaunchKernelGGL((k_pool<float, D>), dim3(pg, BH), dim3(256), 0, ps, (const float*)a.q, a.qs, a.Hq, P.qbar, L, BS);
        hipLaunchKernelGGL((k_pool<float, D>), dim3(pg, bkv), dim3(256), 0, ps, (const float*)a.k, a.ks, a.Hkv, P.kbar, L, BS);
    }
    // K4: the estimated block map needs only the pooled vectors.  At most
    // 22 KB of LDS per workgroup, so that one fits on a CU beside the two
    // score workgroups (64 KB each) running on the other stream: the vector
    // ALU work of the estimate then overlaps their matrix work.
    if (nb <= 1024) {
        const size_t lds = (size_t)4 * nb * sizeof(float);
        hipLaunchKernelGGL((k_estimate<4, D>), dim3((nb + 3) / 4, BH), dim3(256), lds, ps, P.qbar, P.kbar, P.ahat, nb,
                           a.Hq, a.Hkv, group, a.canon);
    } else {
        const size_t lds = (size_t)2 * nb * sizeof(float);
        hipLaunchKernelGGL((k_estimate<2, D>), dim3((nb + 1) / 2, BH), dim3(256), lds, ps, P.qbar, P.kbar, P.ahat, nb,
                           a.Hq, a.Hkv, group, a.canon);
    }
    if (a.aux) {
        he = hipEventRecord(join, ps);
        (void)hipEventDestroy(fork);
        if (he != hipSuccess) {
            // the caller's stream cannot be made to wait: finish the pooling here
            (void)hipStreamSynchronize(a.aux);
            (void)hipEventDestroy(join);
            return he;
        }
    }
    // K2
    const dim3 gs(NS / kScoreTK, BH);
#define FP_SCORES(T, B_)                                                                                   \
    do {                                                                                                   \
        hipLaunchKernelGGL((k_qt<T, B_, D>), dim3(D / 8, BH), dim3(B_), 0, st, (const T*)a.q, a.qs, a.qt, L, a.Hq); \
        if constexpr (sizeof(T) == 2)                                                                      \
            hipLaunchKernelGGL((k_scores_mfma<B_, D>), dim3(scores_mfma_groups(BH, NS / kScoreTK), BH), dim3(256), 0, \
                               st, (const float*)a.qt, (const bf16_t*)a.k, a.ks, a.s2, a.pmax, L, NS, a.Hq, group, \
                               a.canon.C);                                                                 \
        else                                                                                               \
            hipLaunchKernelGGL((k_scores<T, B_, D>), gs, dim3(256), 0, st, (const float*)a.qt, (const T*)a.k, a.ks, \
                               a.s2, a.pmax, L, NS, a.Hq, group, a.canon.C);                               \
    } while (0)
    if (a.dtype_bf16) {
        if (BS == 128) FP_SCORES(bf16_t, 128); else FP_SCORES(bf16_t, 64);
    } else {
        if (BS == 128) FP_SCORES(float, 128); else FP_SCORES(float, 64);
    }
#undef FP_SCORES
    // K3
    if (BS == 128)
        hipLaunchKernelGGL(k_rowexp<128>, dim3(BS, BH), dim3(256), 0, st, a.s2, a.pmax, P.rowmax, P.rowsum, a.rz, L,
                           NS, a.canon);
    else
        hipLaunchKernelGGL(k_rowexp<64>, dim3(BS, BH), dim3(256), 0, st, a.s2, a.pmax, P.rowmax, P.rowsum, a.rz, L,
                           NS, a.canon);
    const int lw = line_width(L, BH);
    const dim3 gl((L + lw - 1) / lw + 1, BH);    // + the diagonal tail's workgroup per head
#define FP_LINESUMS(B_)                                                                                    \
    do {                                                                                                   \
        if (lw == 1024)                                                                                    \
            hipLaunchKernelGGL((k_linesums<B_, 1024>), gl, dim3(256), 0, st, a.s2, P.rowmax, a.rz, P.colsum,  \
                               P.diagsum, P.atrue, L, NS, a.canon);                                        \
        else                                                                                               \
            hipLaunchKernelGGL((k_linesums<B_, 512>), gl, dim3(256), 0, st, a.s2, P.rowmax, a.rz, P.colsum,   \
                               P.diagsum, P.atrue, L, NS, a.canon);                                        \
    } while (0)
    if (BS == 128) FP_LINESUMS(128);
    else FP_LINESUMS(64);
#undef FP_LINESUMS
    // K5
    if (a.aux) {
        he = hipStreamWaitEvent(st, join, 0);
        (void)hipEventDestroy(join);
        if (he != hipSuccess) {
            (void)hipStreamSynchronize(a.aux);
            return he;
        }
    }
    hipLaunchKernelGGL(k_jsd, dim3(BH), dim3(256), 0, st, P.ahat, P.atrue, P.djs, P.pattern, nb, a.tau, a.canon);
    // K6
    const int nlists = 2 * BH;
    if (!P.mode_all) {
        const long long maxlen = P.tri > L ? P.tri : L;
        const int kbits = 31 + index_bits(maxlen);
        const int passes = (kbits + kRadixBits - 1) / kRadixBits;
        if (passes > kSelMaxPasses) return hipErrorInvalidValue;
        hipLaunchKernelGGL(k_sel_reset, dim3(grid1((long long)nlists * kRadixBins)), dim3(256), 0, st, P.sel, P.hist,
                           nlists);
        // list elements per workgroup: every workgroup of a pass first derives
        // the list's state from the previous pass's histogram, so long lists
        // take larger chunks (measured: 4096 at 32k, 8192 at 128k)
        const int chunk = maxlen >= kSelLongList ? 2 * kSelChunk : kSelChunk;
        const dim3 gc((unsigned)((maxlen + chunk - 1) / chunk), nlists);
        hipLaunchKernelGGL(k_sel_total, gc, dim3(256), 0, st, P, P.sel, chunk);
        for (int p = 0; p < passes; ++p)
            hipLaunchKernelGGL(k_sel_pass, gc, dim3(256), 0, st, P, p, nlists, a.G, chunk);
        hipLaunchKernelGGL(k_sel_final, dim3(nlists), dim3(256), 0, st, P, passes, nlists);
        hipLaunchKernelGGL(k_vs_flags, dim3(nb, BH), dim3(BS), 0, st, P, P.sel);
        if (P.cap_blocks > 0) hipLaunchKernelGGL(k_diag_mass, dim3(nb, BH), dim3(64), 0, st, P, P.sel);
    }
    if (P.vs_token) {
        hipLaunchKernelGGL(k_col_scan, dim3(BH), dim3(256), 0, st, P);
        if (!P.mode_all) hipLaunchKernelGGL(k_col_compact, dim3(nb, BH), dim3(BS), 0, st, P, P.sel);
    }
    // K7
    hipLaunchKernelGGL(k_lists, dim3((nb + 3) / 4, BH), dim3(256), 0, st, P, P.sel);
    hipLaunchKernelGGL(k_head_totals, dim3(BH), dim3(256), 0, st, P.counts, P.total_blocks, nb);
    return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, PlanDev& P, hipStream_t st) {
    if (a.d == 128) return launch_plan_t<128>(a, P, st);
    if (a.d == 64) return launch_plan_t<64>(a, P, st);
    return hipErrorInvalidValue;
}

hipError_t launch_fill_u32(unsigned int* p, unsigned int v, long long n, hipStream_t st) {
    if (n > 0) {
        const long long g = (n + 255) / 256;
        hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)(g < 65535 ? g : 65535)), dim3(256), 0, st, p, v, n);
    }
    return hipGetLastError();
}

hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t st) {
    if (bytes % 4 != 0) return hipErrorInvalidValue;
    const unsigned char* s = static_cast<const unsigned char*>(src);
    for (size_t off = 0; off < bytes; off += sizeof(UploadChunk)) {
        UploadChunk c;
        const size_t n = bytes - off < sizeof c ? bytes - off : sizeof c;
        memcpy(c.w, s + off, n);
        hipLaunchKernelGGL(k_upload, dim3(1), dim3(256), 0, st,
                           reinterpret_cast<unsigned int*>(static_cast<unsigned char*>(dst) + off), c, (int)(n / 4));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_zero3_u32(unsigned int* a, long long na, unsigned int* b, long long nb, unsigned int* c,
                           long long nc, hipStream_t st) {
    const long long n = na > nb ? (na > nc ? na : nc) : (nb > nc ? nb : nc);
    if (n > 0) {
        const long long g = (n + 255) / 256;
        hipLaunchKernelGGL(k_zero3_u32, dim3((unsigned)(g < 65535 ? g : 65535), 3), dim3(256), 0, st, a, na, b, nb, c,
                           nc);
    }
    return hipGetLastError();
}

hipError_t launch_probe_exp2(const float* x, float* y, long long n, const Canon& K, hipStream_t st) {
    if (n > 0) hipLaunchKernelGGL(k_probe_exp2, dim3(grid1(n)), dim3(256), 0, st, x, y, n, K);
    return hipGetLastError();
}
hipError_t launch_probe_ln(const double* x, double* y, long long n, const Canon& K, hipStream_t st) {
    if (n > 0) hipLaunchKernelGGL(k_probe_ln, dim3(grid1(n)), dim3(256), 0, st, x, y, n, K);
    return hipGetLastError();
}
hipError_t launch_probe_sqrt(const double* x, double* y, long long n, hipStream_t st) {
    if (n > 0) hipLaunchKernelGGL(k_probe_sqrt, dim3(grid1(n)), dim3(256), 0, st, x, y, n);
    return hipGetLastError();
}

}  // namespace fp
