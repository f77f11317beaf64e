// FlexPrefill step 3 on gfx950: causal flash attention over the key blocks a
// plan selected for each (head, query block) -- the sparse attention the
// pages time against FlashAttention ("Experimental setup" and "Key results"
// of the atlas.scime.ai summary page).  The dense causal variant (every key
// block 0..row) shares the kernel and is the speedup baseline.
//
// Layout of the work: one four-wave workgroup per (head, query block) row at
// block 128, per pair of neighbouring query blocks at block 64; each wave owns
// 32 query rows.  Scores are computed transposed, S^T = K Q^T, with the 32x32
// MFMA: every lane then holds one query's scores for half of a 32-key tile,
// so the row softmax needs a single cross-lane exchange, and the
// probabilities already sit in the B-operand layout of O^T = V^T P^T.  V is
// transposed once per call ([d][N]) so that the V^T A-operand reads are
// contiguous in LDS.  Key tiles of 64 keys are staged through double-buffered
// LDS; grouped-query heads map to kv head h / (Hq / Hkv).  The stage loop is
// software-pipelined: the score MFMAs of the next tile are interleaved with
// the exponentials of the current one, so a wave keeps the matrix unit and
// the vector ALU busy at the same time.
#include <mutex>
#include <vector>

#include "fp_common.h"
#include "fp_launch.h"

namespace fp {

// Workspace of the allocation-free attention entry point (V^T and gathered
// column tiles), one copy per GPU, held until the process ends.  Host code
// never passes `scratch` itself to a kernel: its device address comes from
// hipGetSymbolAddress, taken once per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
    static std::mutex mu;
    static std::vector<void*> addr;   // per device
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    *bytes = kNoAllocScratchBytes;
    return hipSuccess;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kKT = 64;   // keys per LDS stage
constexpr float kLazy = 8.0f;   // log2 growth of a row maximum that forces a rescale
constexpr float kSumLimit = 65536.0f;   // per-lane probability sum that forces a new reference

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// p = exp2(s * sl - mb) for the 32 scores a lane holds, packed as bf16 in
// the B-operand order of O^T += V^T P^T; returns the lane's sum of the
// bf16-rounded values (the same values the numerator uses).
template <int NT>
__device__ __forceinline__ float exp_pack(const f32x16_t (&st)[NT], float sl, float mb, bf16x8_t (&pf)[2 * NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            pf[2 * t + (r >> 3)][r & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(st[t][r], sl, -mb));
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float ls = 0.0f;
#pragma unroll
    for (int kc = 0; kc < 2 * NT; ++kc) {
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[kc], pf[kc], 0, 1), ones, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[kc], pf[kc], 2, 3), ones, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[kc], pf[kc], 4, 5), ones, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[kc], pf[kc], 6, 7), ones, ls, false);
    }
    return ls;
}

// 16 bytes per lane from global memory straight into LDS: a buffer load
// whose resource starts at the (uniform) tile base, plus the lane's 32-bit
// offset.  Lane i's bytes land at dst + 16 i.
__device__ __forceinline__ void lds_load16(const void* base, unsigned voff, void* dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, 0x00020000),
        (__attribute__((address_space(3))) void*)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row of the work handled by workgroup `item`.  Workgroup i of a launch runs
// on XCD i mod 8 whatever the durations (measured with the XCC_ID hardware
// register), so the item order fixes which rows share an XCD's L2 and how
// evenly the XCDs are loaded.
//  - Sparse rows: head after head in the plan's head order (within every
//    group of query heads sharing a key/value head, the heads with the most
//    blocks first, so the launch ends on light heads, and heads reading the
//    same key/value tiles stay adjacent); a head's query blocks descending
//    (longest causal rows first), dealt to the XCDs in chunks of kRowChunk
//    consecutive blocks (kRowChunk / 2 items when a workgroup takes a pair
//    of blocks), so the rows on one XCD share their diagonal and
//    near-diagonal tiles.  Measured on the sparse 128k layer (block 128) and
//    the 64k layer (block 64, 16 query heads per key/value head): chunks of 4
//    blocks take 1 % and 9 % off the attention time against chunks of 1;
//    chunks of 2 or 8 blocks were slower.
//  - Dense rows: the query heads of a key/value group interleaved per query
//    block (with a rotation so every XCD sees every head), so each key/value
//    tile is read by all heads of its group on the same XCD at about the same
//    time (17 % faster at block 64, 1 % at block 128).
//    Interleaving the heads of sparse rows instead measured 2x slower at 128k:
//    heads of different patterns then compete for the L2.
// With several segments (sequences of different lengths) the items of each
// segment follow one another; a workgroup finds its segment by binary
// search in the segment table.
constexpr int kRowChunk = 4;
struct RowId {
    int qb, L, cnt;
    size_t q0, k0, vt0;     // element offsets: token 0 of the query head, of its kv head; its V^T rows
    int NT;                 // V^T row length
    const int* lst;
    int cntB;               // two query blocks per workgroup: the block below qb (count, list)
    const int* lstB;
    int ncol;               // token-granular columns below the row's end (gathered tiles)
    int ncolB;              // ... below the end of the block under qb (pairs)
    const int* gidx;        // the head's selected columns, ascending
    size_t g0;              // element offset of the head's gathered K / V^T
};

__device__ __forceinline__ RowId work_row(const AttnArgs& a, long long item, bool sparse, bool gather = false,
                                          bool pair = false) {
    int lo = 0, hi = a.nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.segs[mid].item0 <= item) lo = mid;
        else hi = mid - 1;
    }
    const AttnSeg sg = a.segs[lo];
    const long long local = item - sg.item0;
    // items per head: one per query block, or one per pair of query blocks
    const int npi = sg.npi;
    int bh, pos;
    if (sparse) {
        const int slot = (int)(local / npi), rr = (int)(local % npi);
        bh = a.hperm ? a.hperm[sg.hoff + slot] - (int)sg.hoff : slot;
        const int C = pair ? kRowChunk / 2 : kRowChunk, C8 = 8 * C;   // items per chunk
        const int blk = rr / C8, within = rr % C8;
        pos = (blk + 1) * C8 <= npi ? blk * C8 + (within % 8) * C + within / 8 : rr;
    } else {
        const int G = a.Hq / a.Hkv;
        const long long gsz = (long long)G * npi;
        const int grp = (int)(local / gsz), u = (int)(local % gsz);
        pos = u / G;
        const int rot = pos / (G >= 8 ? 1 : 8 / G);
        bh = (grp / a.Hkv) * a.Hq + (grp % a.Hkv) * G + (u % G + rot) % G;
    }
    RowId r;
    r.qb = sg.nb - 1 - (pair ? 2 * pos : pos);
    r.L = sg.L;
    r.NT = sg.NT;
    const int bl = bh / a.Hq, h = bh % a.Hq, kvh = h / (a.Hq / a.Hkv);
    r.q0 = (size_t)sg.qoff + (size_t)bl * a.qs.bst + (size_t)h * a.qs.hs;
    r.k0 = (size_t)sg.koff + (size_t)bl * a.ks.bst + (size_t)kvh * a.ks.hs;
    r.vt0 = (size_t)sg.vtoff + (size_t)(bl * a.Hkv + kvh) * a.d * sg.NT;
    if (sparse) {
        const long long tri = (long long)sg.nb * (sg.nb + 1) / 2;
        r.cnt = a.counts[sg.coff + (long long)bh * sg.nb + r.qb];
        r.lst = a.lists + sg.loff + (long long)bh * tri + (long long)r.qb * (r.qb + 1) / 2;
        const int qbB = r.qb - 1;
        r.cntB = pair && qbB >= 0 ? a.counts[sg.coff + (long long)bh * sg.nb + qbB] : 0;
        r.lstB = pair && qbB >= 0 ? a.lists + sg.loff + (long long)bh * tri + (long long)qbB * (qbB + 1) / 2 : r.lst;
    } else {
        r.cnt = r.qb + 1;
        r.lst = nullptr;
        r.cntB = r.qb;
        r.lstB = nullptr;
    }
    r.ncol = 0;
    r.ncolB = 0;
    r.gidx = nullptr;
    r.g0 = 0;
    if (gather) {
        const int* cp = a.colptr + sg.cpoff + (long long)bh * (sg.nb + 1);
        r.ncol = cp[r.qb + 1];
        r.ncolB = pair && r.qb >= 1 ? cp[r.qb] : 0;
        r.gidx = a.colidx + sg.cioff + (long long)bh * sg.L;
        r.g0 = (size_t)sg.goff + (size_t)bh * a.d * sg.NT;
    }
    return r;
}

// Mask of a gathered-column tile (64 keys, one per lane: column c = 64 t +
// lane of the head's ascending selected columns): a key is dropped when it
// lies past the row's columns, inside one of the row's full blocks (those
// are attended in full already) or, in the diagonal block, after the query.
// Each wave writes the tile's additive bias (0 or -inf) and, for keys in the
// diagonal block, their positions to its own LDS slot; every lane then adds
// the biases of its 32 keys with 16-byte reads.
template <int BS>
__device__ __forceinline__ void gather_mask(f32x16_t (&st)[2], int t, const RowId& rid, int ncol,
                                            const unsigned int* fbits, float* gb, int* gj, int qb, int qrow, int lane,
                                            int hh) {
    const int c = 64 * t + lane;
    const int j = c < ncol ? rid.gidx[c] : -1;
    const int jb = j >= 0 ? j / BS : 0;
    const bool valid = j >= 0 && !((fbits[jb >> 5] >> (jb & 31)) & 1u);
    const bool diag = valid && jb == qb;
    gb[lane] = valid ? 0.0f : -INFINITY;
    gj[lane] = diag ? j : -1;
    const bool anydiag = __ballot(diag) != 0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(&gb[32 * u + 8 * q + 4 * hh]);
#pragma unroll
            for (int e = 0; e < 4; ++e) st[u][4 * q + e] += bv[e];
        }
    if (anydiag) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int4 jv = *reinterpret_cast<const int4*>(&gj[32 * u + 8 * q + 4 * hh]);
                if (jv.x > qrow) st[u][4 * q] = -INFINITY;
                if (jv.y > qrow) st[u][4 * q + 1] = -INFINITY;
                if (jv.z > qrow) st[u][4 * q + 2] = -INFINITY;
                if (jv.w > qrow) st[u][4 * q + 3] = -INFINITY;
            }
    }
    __builtin_amdgcn_wave_barrier();   // the slot is rewritten by the next tile
}

// ---------------------------------------------------------------------------
// bf16 inputs, bf16 MFMA 32x32x16, fp32 accumulation and softmax
// ---------------------------------------------------------------------------
// Stages of 64 keys.  Block 128: one four-wave workgroup per query block, two
// workgroups per CU.  PAIR (block 64; dense rows at block 128): one workgroup
// takes two neighbouring query blocks of a head (the first half of its waves
// block qb, the second half block qb - 1) and walks the union of their lists:
// each key/value tile is loaded once for twice the queries, and a wave skips
// the P V work of the tiles its own row's list lacks.  With gathered token
// columns the pair walks the column tiles of block qb and each wave masks the
// columns past its own row.  Two workgroups per CU, one for the eight-wave
// block-128 pairs.
template <int BS, bool SPARSE, bool GATHER, bool PAIR, int D>
__global__ __launch_bounds__(PAIR ? 2 * 2 * BS : 2 * BS, (PAIR && BS == 128) ? 1 : 2) void k_attn_bf16(AttnArgs a) {
    constexpr int KT = kKT, NW = PAIR ? 2 * (BS / 32) : BS / 32, SPB = BS / KT;
    constexpr int NTH = 64 * NW;                // threads
    constexpr int NT = KT / 32;                 // 32-key score tiles per stage
    constexpr int QC = D / 16;                  // 16-wide contraction chunks of a score tile
    constexpr int TDV = D / 32;                 // 32-row dv tiles of O^T
    constexpr int NMS = QC * NT;                // score MFMAs per stage
    constexpr int EPS = 16 * NT / NMS;          // exponentials per score MFMA (32 per lane per stage)
    constexpr int NMV = TDV * 2 * NT;           // P V MFMAs per stage
    constexpr int KCH = D / 8;                  // 16-byte chunks per K row
    constexpr int RPL = 1024 / (2 * D);         // K rows per 1 KB load
    static_assert(EPS % 2 == 0 && 32 % KCH == 0, "tile layout");
    constexpr int CPR = KT / 8;                 // 16-byte chunks per V^T row
    constexpr int TILE = KT * D * 2;            // bytes of one K (or V^T) tile
    constexpr int LOADS = TILE / 1024 / NW;     // 1 KB loads into LDS per wave per tile
    static_assert(LOADS >= 1 && TILE % (1024 * NW) == 0, "tile loads");
    // Tiles are unpadded and XOR-swizzled at 16-byte granularity:
    //   K   [KT keys][2 D bytes]:  chunk c of row r at chunk c ^ (r & (KCH - 1))
    //   V^T [128 dv][2 KT bytes]:  chunk c of row r at chunk c ^ gray(r) & (CPR - 1)
    // so that the MFMA fragment reads below hit distinct banks.
    // The tiles are four separate LDS objects and the stage loop is unrolled
    // by two, so every access names its buffer at compile time: the compiler
    // can then tell that the loads filling one buffer do not alias the reads
    // of another, and the tile loads stay in flight during the whole stage.
    // The loads are buffer loads (not global ones): with a global load into
    // LDS in flight the compiler waits for every outstanding LDS read instead
    // of only the one an MFMA needs.
    __shared__ __attribute__((aligned(1024))) unsigned char Ks0[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char Ks1[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char Vs0[TILE];
    __shared__ __attribute__((aligned(1024))) unsigned char Vs1[TILE];
    __shared__ unsigned int fbits[GATHER && !PAIR ? kMaxBlocks / 32 : 1];   // the row's full blocks
    __shared__ __attribute__((aligned(16))) float gbias[GATHER ? NW : 1][64];
    __shared__ __attribute__((aligned(16))) int gjpos[GATHER ? NW : 1][64];
    // PAIR, sparse: each row's blocks as bits, the union of the two lists ascending
    constexpr bool UNION = PAIR && SPARSE;
    static_assert(!UNION || kMaxBlocks == 64 * 64, "one wave scans the block bitmaps");
    __shared__ unsigned int pbits[UNION ? 2 : 1][UNION ? kMaxBlocks / 32 : 1];
    __shared__ unsigned short ulist[UNION ? kMaxBlocks : 1];
    __shared__ int ucnt[1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
    const int l32 = lane & 31, hh = lane >> 5;
    const RowId rid = work_row(a, blockIdx.x, SPARSE, GATHER, PAIR);
    // PAIR: the wave's query block, -1 for the missing partner of block 0
    const int prow = PAIR ? (w / (BS / 32)) : 0;
    const int qb = rid.qb - prow, L = rid.L;
    const unsigned char* K = (const unsigned char*)a.k + rid.k0 * 2;
    const unsigned char* VT = (const unsigned char*)a.vt + rid.vt0 * 2;
    const size_t vrow = (size_t)rid.NT * 2;      // bytes per V^T row
    const size_t krs = (size_t)a.ks.rs * 2;      // bytes per key row

    const int cnt = rid.cnt;
    // the row's list is read with scalar loads (uniform addresses, counted
    // apart from the vector-memory tile loads)
    typedef const __attribute__((address_space(4))) int* cint_p;
    const cint_p lst = (cint_p)rid.lst;
    int nsub = cnt * SPB;
    // token-granular columns: 64-key tiles of the head's gathered K / V^T after
    // the blocks (a pair walks those of block qb, whose columns include those
    // of qb - 1; each wave masks the columns past its own row)
    const int ngs = GATHER ? (rid.ncol + KT - 1) / KT : 0;
    const int ncolW = prow ? rid.ncolB : rid.ncol;
    (void)ncolW;
    int nstage = nsub + ngs;
    if constexpr (UNION) {
        const cint_p lstB = (cint_p)rid.lstB;
        for (int e = tid; e < 2 * kMaxBlocks / 32; e += NTH) (&pbits[0][0])[e] = 0u;
        __syncthreads();
        for (int e = tid; e < cnt; e += NTH) atomicOr(&pbits[0][lst[e] >> 5], 1u << (lst[e] & 31));
        for (int e = tid; e < rid.cntB; e += NTH) atomicOr(&pbits[1][lstB[e] >> 5], 1u << (lstB[e] & 31));
        __syncthreads();
        if (w == 0) {
            // lane l: blocks 64 l .. 64 l + 63; exclusive scan of the union counts
            const unsigned a0 = pbits[0][2 * lane], b0 = pbits[1][2 * lane];
            const unsigned a1 = pbits[0][2 * lane + 1], b1 = pbits[1][2 * lane + 1];
            const unsigned u0 = a0 | b0, u1 = a1 | b1;
            const int c = __popc(u0) + __popc(u1);
            int incl = c;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o);
                if (lane >= o) incl += t;
            }
            int at = incl - c;
            // entry: key block | in the list of block qb (bit 12) | of block qb - 1 (bit 13)
            for (unsigned m = u0; m; m &= m - 1) {
                const int t = __builtin_ctz(m);
                ulist[at++] = (unsigned short)((64 * lane + t) | ((a0 >> t) & 1u) << 12 | ((b0 >> t) & 1u) << 13);
            }
            for (unsigned m = u1; m; m &= m - 1) {
                const int t = __builtin_ctz(m);
                ulist[at++] = (unsigned short)((64 * lane + 32 + t) | ((a1 >> t) & 1u) << 12 | ((b1 >> t) & 1u) << 13);
            }
            if (lane == 63) ucnt[0] = incl;
        }
        __syncthreads();
        nsub = __builtin_amdgcn_readfirstlane(ucnt[0]) * SPB;
        nstage = nsub + ngs;
    } else if constexpr (PAIR) {
        nsub = nstage = (rid.qb + 1) * SPB;
    }
    // Union walks keep the list entries of stages s, s + 1 and s + 2 in scalar
    // registers (uwin) and read the entry of stage s + 3 from LDS during stage
    // s, so no tile load waits on an LDS read for its address.
    const int ulast = UNION ? (nsub > 0 ? nsub / SPB - 1 : 0) : 0;
    int uwin[3] = {0, 0, 0};
    if constexpr (UNION) {
#pragma unroll
        for (int i = 0; i < 3; ++i) uwin[i] = __builtin_amdgcn_readfirstlane((int)ulist[min(i / SPB, ulast)]);
    }
    // key block of stage s_ (for union walks s_ is s_cur, s_cur + 1 or
    // s_cur + 2, s_cur being the stage in progress), and whether a block is in
    // this wave's own list
#define FP_KB(s_) (UNION ? (uwin[(s_) - s_cur] & 4095)                                                     \
                         : (PAIR ? (s_) / SPB : (SPARSE ? lst[(s_) / SPB] : (s_) / SPB)))
#define FP_MINE(kb_) (!PAIR || (kb_) <= qb)
    const unsigned char* KG = GATHER ? (const unsigned char*)a.kg + rid.g0 * 2 : nullptr;
    const unsigned char* VGT = GATHER ? (const unsigned char*)a.vgt + rid.g0 * 2 : nullptr;
    if (GATHER && !PAIR && ngs > 0) {
        for (int e = tid; e < kMaxBlocks / 32; e += NTH) fbits[e] = 0u;
        __syncthreads();
        for (int e = tid; e < cnt; e += NTH) atomicOr(&fbits[lst[e] >> 5], 1u << (lst[e] & 31));
        __syncthreads();
    }

    // Q fragments (B operand of S^T = K Q^T): query l32 of this wave, d = 16c + 8hh + [0, 8).
    // Rows past the sequence end (a partial last block) read its last row and are not stored.
    const int qrel = 32 * (PAIR ? (w % (BS / 32)) : w) + l32;
    const int qrow = qb * BS + qrel;
    bf16x8_t qf[QC];
    {
        const bf16_t* qp = (const bf16_t*)a.q + rid.q0 + (size_t)max(min(qrow, L - 1), 0) * a.qs.rs + 8 * hh;
#pragma unroll
        for (int c = 0; c < QC; ++c) qf[c] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * c);
    }

    f32x16_t o[TDV];
#pragma unroll
    for (int T = 0; T < TDV; ++T)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[T][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    const float sl = a.scale_log2;

    // Per-lane source offsets of the tile loads (independent of the stage).
    // K load j of wave w covers rows RPL J .. RPL J + RPL - 1 (J = w + NW j); lane -> row
    // RPL J + lane / KCH, stored chunk lane % KCH holds logical chunk (lane % KCH) ^ (row % KCH).
    // V^T load j covers rows (64/CPR) J ..; lane -> row (64/CPR) J + lane/CPR, stored
    // chunk lane%CPR holds logical chunk (lane%CPR) ^ gray(row) & (CPR-1).
    unsigned koff[LOADS], voff[LOADS];
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
        const int J = w + NW * j;
        const int kr = RPL * J + lane / KCH;
        koff[j] = (unsigned)(kr * krs + 16 * ((lane % KCH) ^ (kr & (KCH - 1))));
        const int vr = (64 / CPR) * J + lane / CPR;
        voff[j] = (unsigned)((size_t)vr * vrow + 16 * ((lane % CPR) ^ ((vr ^ (vr >> 1)) & (CPR - 1))));
    }
    // Tiles go straight from global memory to LDS (buffer loads with the
    // tile's first byte as the uniform base and the offsets above per lane).
    // A tile reaching past the sequence end (only in the last key block) reads
    // the last key for the missing rows: finite values that the causal mask
    // removes; V^T is zero there.
#define FP_FETCH_K(s_, KD_)                                                                              \
    {                                                                                                    \
        if (!GATHER || (s_) < nsub) {                                                                    \
            const int kb_ = FP_KB(s_);                                                                  \
            const int key0_ = kb_ * BS + ((s_) % SPB) * KT;                                             \
            const unsigned char* kg_ = K + (size_t)key0_ * krs;                                         \
            if (key0_ + KT <= L) {                                                                      \
                _Pragma("unroll") for (int j = 0; j < LOADS; ++j)                                       \
                    lds_load16(kg_, koff[j], &KD_[(w + NW * j) * 1024]);                               \
            } else {                                                                                    \
                _Pragma("unroll") for (int j = 0; j < LOADS; ++j) {                                     \
                    const int kr_ = RPL * (w + NW * j) + lane / KCH;                                    \
                    const unsigned o_ = (unsigned)((min(key0_ + kr_, L - 1) - key0_) * krs) +           \
                                        16u * ((lane % KCH) ^ (kr_ & (KCH - 1)));                       \
                    lds_load16(kg_, o_, &KD_[(w + NW * j) * 1024]);                                    \
                }                                                                                       \
            }                                                                                           \
        } else {                                                                                         \
            const unsigned char* kg_ = KG + (size_t)((s_) - nsub) * KT * D * 2;                         \
            _Pragma("unroll") for (int j = 0; j < LOADS; ++j) {                                         \
                const int kr_ = RPL * (w + NW * j) + lane / KCH;                                        \
                lds_load16(kg_, (unsigned)(kr_ * D * 2 + 16 * ((lane % KCH) ^ (kr_ & (KCH - 1)))),     \
                            &KD_[(w + NW * j) * 1024]);                                                 \
            }                                                                                           \
        }                                                                                                \
    }
#define FP_FETCH_V(s_, VD_)                                                                              \
    {                                                                                                    \
        const unsigned char* vg_;                                                                        \
        if (!GATHER || (s_) < nsub) {                                                                    \
            const int kb_ = FP_KB(s_);                                                                  \
            vg_ = VT + (size_t)(kb_ * BS + ((s_) % SPB) * KT) * 2;                                      \
        } else {                                                                                         \
            vg_ = VGT + (size_t)(((s_) - nsub) * KT) * 2;                                               \
        }                                                                                                \
        _Pragma("unroll") for (int j = 0; j < LOADS; ++j)                                               \
            lds_load16(vg_, voff[j], &VD_[(w + NW * j) * 1024]);                                       \
    }
    // Operand fragments in LDS: K rows (S^T = K Q^T) and V^T rows (O^T += V^T P^T).
#define FP_KFRAG(B_, t_, c_) (*reinterpret_cast<const bf16x8_t*>(&B_[kfa[(c_)] + (t_) * 32 * D * 2]))
#define FP_VFRAG(B_, T_, kc_) (*reinterpret_cast<const bf16x8_t*>(                                       \
        &B_[(32 * (T_) + l32) * KT * 2 +                                                                \
             16 * ((2 * (kc_) + hh) ^ (((32 * (T_) + l32) ^ ((32 * (T_) + l32) >> 1)) & (CPR - 1)))]))
    // byte offset of K fragment c (contraction chunk c) of key row l32 within a
    // 32-row half tile; the half (t) and the buffer are immediate offsets
    unsigned kfa[QC];
#pragma unroll
    for (int c = 0; c < QC; ++c) kfa[c] = (unsigned)(l32 * D * 2 + 16 * ((2 * c + hh) ^ (l32 & (KCH - 1))));
    constexpr int RING = 4;   // LDS operand reads in flight ahead of the MFMAs
    const f32x16_t zero16 = {};

    // Software pipeline: stage s runs the softmax of tile s while the matrix
    // unit computes the scores of tile s + 1, then O^T += V^T P^T of tile s.
    // K tiles are fetched two stages ahead, V^T tiles one stage ahead.
    f32x16_t scA[NT], scB[NT];
    {
        const int s_cur = 0;
        (void)s_cur;
        FP_FETCH_K(0, Ks0);
        FP_FETCH_V(0, Vs0);
        if (nstage > 1) { FP_FETCH_K(1, Ks1); }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NMS; ++i)
        scA[i % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FP_KFRAG(Ks0, i % NT, i / NT), qf[i / NT],
                                                              i < NT ? zero16 : scA[i % NT], 0, 0, 0);
    __syncthreads();

    // One stage.  The 16 score MFMAs of the next tile are interleaved with
    // the exponentials of this tile (two scores per MFMA); scheduling fences
    // keep that order, so each MFMA runs while the vector ALU works.  With
    // query-block pairs the exponentials feed only the tiles of the wave's own
    // list, so the compiler moves them behind that test, after the MFMAs:
    // there that schedule measured as fast as the interleave or 1-3 % faster
    // (the interleave costs clock under the power cap), while one query block
    // per workgroup runs 8 % slower without the interleave.
#define FP_STAGE_BF16(s, KC_, VC_, KN_, VN_, SC_, SN_)                                                   \
    {                                                                                                    \
        const int s_cur = (s);                                                                           \
        (void)s_cur;                                                                                     \
        const bool gst = GATHER && (s) >= nsub;                                                          \
        const int kb = gst ? -1 : FP_KB(s);                                                              \
        const int sub = (s) % SPB;                                                                       \
        const int uvn = UNION ? (int)ulist[min(((s) + 3) / SPB, ulast)] : 0;                             \
        if ((s) + 2 < nstage) { FP_FETCH_K((s) + 2, KN_); }                                              \
        if ((s) + 1 < nstage) { FP_FETCH_V((s) + 1, VN_); }                                              \
        /* PAIR: a tile outside the wave's own list gets scores and exponentials */                     \
        /* (cheap: the union exceeds each list by a few tiles) but no P V and no row sum */              \
        const bool mS = gst || (UNION ? ((uwin[0] >> (12 + prow)) & 1) != 0 : FP_MINE(kb));            \
        if (kb == qb) {                                                                                  \
            _Pragma("unroll") for (int t = 0; t < NT; ++t)                                               \
            _Pragma("unroll") for (int r = 0; r < 16; ++r) {                                             \
                const int krel = sub * KT + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);                   \
                if (krel > qrel) SC_[t][r] = -INFINITY;                                                  \
            }                                                                                            \
        }                                                                                                \
        if constexpr (GATHER) {                                                                          \
            if (gst) gather_mask<BS>(SC_, (s) - nsub, rid, PAIR ? ncolW : rid.ncol, PAIR ? pbits[prow] : fbits, \
                                     gbias[w], gjpos[w], qb, qrow, lane, hh);                            \
        }                                                                                                \
        bf16x8_t pf[2 * NT];                                                                             \
        float ls = 0.0f;                                                                                 \
        const float mb = m_run * sl;                                                                     \
        {                                                                                                \
            bf16x8_t fr[RING];                                                                           \
            _Pragma("unroll") for (int i = 0; i < RING; ++i) fr[i] = FP_KFRAG(KC_, i % NT, i / NT);      \
            __builtin_amdgcn_sched_barrier(0);                                                           \
            _Pragma("unroll") for (int i = 0; i < NMS; ++i) {                                            \
                SN_[i % NT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % RING], qf[i / NT],          \
                                                                      i < NT ? zero16 : SN_[i % NT], 0, 0, 0); \
                if (i + RING < NMS) fr[i % RING] = FP_KFRAG(KC_, (i + RING) % NT, (i + RING) / NT);     \
                _Pragma("unroll") for (int u_ = 0; u_ < EPS / 2; ++u_) {                                 \
                    const int x_ = EPS * i + 2 * u_, t_ = x_ >> 4, r_ = x_ & 15;                         \
                    const float e0_ = __builtin_amdgcn_exp2f(__builtin_fmaf(SC_[t_][r_], sl, -mb));      \
                    const float e1_ = __builtin_amdgcn_exp2f(__builtin_fmaf(SC_[t_][r_ + 1], sl, -mb));  \
                    const bf16x2_t p2_ = {(__bf16)e0_, (__bf16)e1_};                                     \
                    pf[2 * t_ + (r_ >> 3)][r_ & 7] = p2_[0];                                             \
                    pf[2 * t_ + (r_ >> 3)][(r_ & 7) + 1] = p2_[1];                                       \
                    ls = __builtin_amdgcn_fdot2_f32_bf16(p2_, ones2, ls, false);                          \
                }                                                                                        \
                __builtin_amdgcn_sched_barrier(0);                                                       \
            }                                                                                            \
        }                                                                                                \
        if (mS) {                                                                                        \
            if (__ballot(!(ls <= kSumLimit)) != 0) {                                                     \
                float mx = -INFINITY;                                                                    \
                _Pragma("unroll") for (int t = 0; t < NT; ++t)                                           \
                _Pragma("unroll") for (int r = 0; r < 16; ++r) mx = fmaxf(mx, SC_[t][r]);                \
                mx = fmaxf(mx, __shfl_xor(mx, 32));                                                      \
                const float m_new = fmaxf(m_run, mx);                                                    \
                const float alpha = fast_exp2((m_run - m_new) * sl);                                     \
                l_run *= alpha;                                                                          \
                _Pragma("unroll") for (int T = 0; T < TDV; ++T)                                          \
                _Pragma("unroll") for (int r = 0; r < 16; ++r) o[T][r] *= alpha;                         \
                m_run = m_new;                                                                           \
                ls = exp_pack(SC_, sl, m_run * sl, pf);                                                  \
            }                                                                                            \
            l_run += ls;                                                                                 \
            bf16x8_t fr[RING];                                                                           \
            _Pragma("unroll") for (int i = 0; i < RING; ++i) fr[i] = FP_VFRAG(VC_, i % TDV, i / TDV);    \
            __builtin_amdgcn_sched_barrier(0);                                                           \
            _Pragma("unroll") for (int i = 0; i < NMV; ++i) {                                            \
                o[i % TDV] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % RING], pf[i / TDV], o[i % TDV], 0, 0, 0); \
                if (i + RING < NMV) fr[i % RING] = FP_VFRAG(VC_, (i + RING) % TDV, (i + RING) / TDV);    \
                __builtin_amdgcn_sched_barrier(0);                                                       \
            }                                                                                            \
        }                                                                                                \
        if constexpr (UNION) {                                                                           \
            uwin[0] = uwin[1];                                                                           \
            uwin[1] = uwin[2];                                                                           \
            uwin[2] = __builtin_amdgcn_readfirstlane(uvn);                                               \
        }                                                                                                \
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");                                                 \
        __syncthreads();                                                                                 \
    }

    // online softmax (lane = one query; lane ^ 32 holds its other keys).
    // The exp2 arguments use the reference maximum of earlier stages; as
    // long as every lane's sum of the new probabilities stays <= kSumLimit
    // (so each is <= kSumLimit) that reference is kept and no maximum is
    // formed at all.  Otherwise (always on the first stage, whose reference
    // -inf makes every sum infinite or NaN) the exact maximum becomes the
    // reference, the accumulators are rescaled and the probabilities
    // recomputed.  The final division by the row sum makes the result
    // independent of the reference chosen.  O^T += V^T P^T uses the key order
    // kc*16 + 8*(e/4) + 4*hh + e%4 of the B operand; V^T rows store each
    // 16-key chunk as key groups [0-3, 8-11, 4-7, 12-15], so those 8 keys are
    // one contiguous 16-byte chunk (logical chunk 2kc + hh).
    // Stage s reads K(s+1) from buffer (s+1)%2 and V(s) from buffer s%2, and
    // fills K(s+2) into buffer s%2 and V(s+1) into buffer (s+1)%2; on the
    // last stage the score MFMAs read a stale tile and their result is unused.
    const bf16x2_t ones2 = {(__bf16)1.0f, (__bf16)1.0f};
    for (int s = 0; s < nstage; s += 2) {
        FP_STAGE_BF16(s, Ks1, Vs0, Ks0, Vs1, scA, scB);
        if (s + 1 < nstage) FP_STAGE_BF16(s + 1, Ks0, Vs1, Ks1, Vs0, scB, scA);
    }
#undef FP_STAGE_BF16
#undef FP_KB
#undef FP_MINE
#undef FP_KFRAG
#undef FP_VFRAG
#undef FP_FETCH_K
#undef FP_FETCH_V

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    if (qb < 0 || qrow >= L) return;
    bf16_t* op = (bf16_t*)a.o + rid.q0 + (size_t)qrow * a.qs.rs;
#pragma unroll
    for (int T = 0; T < TDV; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dv = 32 * T + 8 * i + 4 * hh;
            ushort4 pk;
            pk.x = f32_to_bf16(o[T][4 * i] * inv);
            pk.y = f32_to_bf16(o[T][4 * i + 1] * inv);
            pk.z = f32_to_bf16(o[T][4 * i + 2] * inv);
            pk.w = f32_to_bf16(o[T][4 * i + 3] * inv);
            *reinterpret_cast<ushort4*>(op + dv) = pk;
        }
}

// ---------------------------------------------------------------------------
// fp32 inputs: fp32 MFMA 32x32x2, same structure.  Contraction index e of a
// lane pair (hh) maps to d = c + (D / 2) hh (scores) and to key 32t + 8i + 4hh + j
// (values), identically for both operands.
// ---------------------------------------------------------------------------
template <int BS, bool SPARSE, bool GATHER, int D>
__global__ __launch_bounds__(2 * BS) void k_attn_f32(AttnArgs a) {
    constexpr int KT = kKT, NT = 2 * BS, SPB = BS / KT, HD = D / 2, TDV = D / 32, D4 = D / 4;
    constexpr int KP = D + 4;     // floats: 528 B
    constexpr int VP = KT + 4;    // floats: 272 B
    constexpr int KCH = KT * D / 4 / NT;
    constexpr int VCH = D * KT / 4 / NT;
    extern __shared__ __attribute__((aligned(16))) float smem_f32[];
    float* Ks0 = smem_f32;
    float* Vs0 = smem_f32 + 2 * KT * KP;

    __shared__ unsigned int fbits[GATHER ? kMaxBlocks / 32 : 1];   // the row's full blocks
    __shared__ __attribute__((aligned(16))) float gbias[GATHER ? BS / 32 : 1][64];
    __shared__ __attribute__((aligned(16))) int gjpos[GATHER ? BS / 32 : 1][64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l32 = lane & 31, hh = lane >> 5;
    const RowId rid = work_row(a, blockIdx.x, SPARSE, GATHER);
    const int qb = rid.qb, L = rid.L;
    const float* K = (const float*)a.k + rid.k0;
    const float* VT = (const float*)a.vt + rid.vt0;
    const size_t krs = (size_t)a.ks.rs;
    const size_t NTv = (size_t)rid.NT;

    const int cnt = rid.cnt;
    const int* lst = rid.lst;
    const int nsub = cnt * SPB;
    const int ngs = GATHER ? (rid.ncol + KT - 1) / KT : 0;
    const int nstage = nsub + ngs;
    const float* KG = GATHER ? (const float*)a.kg + rid.g0 : nullptr;
    const float* VGT = GATHER ? (const float*)a.vgt + rid.g0 : nullptr;
    if (GATHER && ngs > 0) {
        for (int e = tid; e < kMaxBlocks / 32; e += NT) fbits[e] = 0u;
        __syncthreads();
        for (int e = tid; e < cnt; e += NT) atomicOr(&fbits[lst[e] >> 5], 1u << (lst[e] & 31));
        __syncthreads();
    }
    const int qrel = 32 * w + l32;
    const int qrow = qb * BS + qrel;
    float qf[HD];
    {
        const float* qp = (const float*)a.q + rid.q0 + (size_t)min(qrow, L - 1) * a.qs.rs + HD * hh;
#pragma unroll
        for (int c = 0; c < HD; c += 4) {
            const float4 v = *reinterpret_cast<const float4*>(qp + c);
            qf[c] = v.x; qf[c + 1] = v.y; qf[c + 2] = v.z; qf[c + 3] = v.w;
        }
    }
    f32x16_t o[TDV];
#pragma unroll
    for (int T = 0; T < TDV; ++T)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[T][r] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    const float sl = a.scale_log2;

    f32x4_t kreg[KCH], vreg[VCH];
#define FP_FETCH_F32(s_)                                                                             \
    if (!GATHER || (s_) < nsub) {                                                                    \
        const int kb_ = SPARSE ? lst[(s_) / SPB] : (s_) / SPB;                                          \
        const int key0_ = kb_ * BS + ((s_) % SPB) * KT;                                              \
        _Pragma("unroll") for (int r = 0; r < KCH; ++r) {                                            \
            const int e = tid + NT * r, key = e / D4, d4 = e % D4;                                   \
            kreg[r] = *reinterpret_cast<const f32x4_t*>(K + (size_t)min(key0_ + key, L - 1) * krs + 4 * d4); \
        }                                                                                            \
        _Pragma("unroll") for (int r = 0; r < VCH; ++r) {                                            \
            const int e = tid + NT * r, dv = e >> 4, k4 = e & 15;                                    \
            vreg[r] = *reinterpret_cast<const f32x4_t*>(VT + (size_t)dv * NTv + key0_ + 4 * k4);      \
        }                                                                                            \
    } else {                                                                                         \
        const int c0_ = ((s_) - nsub) * KT;                                                          \
        _Pragma("unroll") for (int r = 0; r < KCH; ++r) {                                            \
            const int e = tid + NT * r, key = e / D4, d4 = e % D4;                                   \
            kreg[r] = *reinterpret_cast<const f32x4_t*>(KG + (size_t)(c0_ + key) * D + 4 * d4);      \
        }                                                                                            \
        _Pragma("unroll") for (int r = 0; r < VCH; ++r) {                                            \
            const int e = tid + NT * r, dv = e >> 4, k4 = e & 15;                                    \
            vreg[r] = *reinterpret_cast<const f32x4_t*>(VGT + (size_t)dv * NTv + c0_ + 4 * k4);      \
        }                                                                                            \
    }
#define FP_STASH_F32(buf_)                                                                           \
    {                                                                                                \
        float* Ks_ = Ks0 + (buf_) * KT * KP;                                                         \
        float* Vs_ = Vs0 + (buf_) * D * VP;                                                          \
        _Pragma("unroll") for (int r = 0; r < KCH; ++r) {                                            \
            const int e = tid + NT * r, key = e / D4, d4 = e % D4;                                   \
            *reinterpret_cast<f32x4_t*>(&Ks_[key * KP + 4 * d4]) = kreg[r];                           \
        }                                                                                            \
        _Pragma("unroll") for (int r = 0; r < VCH; ++r) {                                            \
            const int e = tid + NT * r, dv = e >> 4, k4 = e & 15;                                    \
            *reinterpret_cast<f32x4_t*>(&Vs_[dv * VP + 4 * k4]) = vreg[r];                            \
        }                                                                                            \
    }

    FP_FETCH_F32(0);
    FP_STASH_F32(0);
    __syncthreads();
    for (int s = 0; s < nstage; ++s) {
        const int buf = s & 1;
        const float* Ks = Ks0 + buf * KT * KP;
        const float* Vs = Vs0 + buf * D * VP;
        const bool gst = GATHER && s >= nsub;
        const int kb = gst ? -1 : (SPARSE ? lst[s / SPB] : s / SPB);
        const int sub = s % SPB;
        if (s + 1 < nstage) { FP_FETCH_F32(s + 1); }
        f32x16_t st[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int r = 0; r < 16; ++r) st[t][r] = 0.0f;
            const float* kr = &Ks[(32 * t + l32) * KP + HD * hh];
#pragma unroll
            for (int c = 0; c < HD; c += 4) {
                const float4 kv = *reinterpret_cast<const float4*>(kr + c);
                st[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.x, qf[c], st[t], 0, 0, 0);
                st[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.y, qf[c + 1], st[t], 0, 0, 0);
                st[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.z, qf[c + 2], st[t], 0, 0, 0);
                st[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.w, qf[c + 3], st[t], 0, 0, 0);
            }
        }
        if (kb == qb) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int krel = sub * KT + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (krel > qrel) st[t][r] = -INFINITY;
                }
        }
        if (GATHER && gst) gather_mask<BS>(st, s - nsub, rid, rid.ncol, fbits, gbias[w], gjpos[w], qb, qrow, lane, hh);
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[t][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool grow = !(m_run * sl + kLazy >= mx * sl);
        if (__ballot(grow)) {
            const float m_new = grow ? fmaxf(m_run, mx) : m_run;
            const float alpha = fast_exp2((m_run - m_new) * sl);
            l_run *= alpha;
#pragma unroll
            for (int T = 0; T < TDV; ++T)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[T][r] *= alpha;
            m_run = m_new;
        }
        const float mb = m_run == -INFINITY ? 0.0f : m_run * sl;
        float ls = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                st[t][r] = fast_exp2(__builtin_fmaf(st[t][r], sl, -mb));
                ls += st[t][r];
            }
        l_run += ls;
#pragma unroll
        for (int T = 0; T < TDV; ++T) {
            const float* vr = &Vs[(32 * T + l32) * VP + 4 * hh];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 vv = *reinterpret_cast<const float4*>(vr + 32 * t + 8 * i);
                    o[T] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.x, st[t][4 * i], o[T], 0, 0, 0);
                    o[T] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.y, st[t][4 * i + 1], o[T], 0, 0, 0);
                    o[T] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.z, st[t][4 * i + 2], o[T], 0, 0, 0);
                    o[T] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.w, st[t][4 * i + 3], o[T], 0, 0, 0);
                }
        }
        if (s + 1 < nstage) FP_STASH_F32(buf ^ 1);
        __syncthreads();
    }
#undef FP_FETCH_F32
#undef FP_STASH_F32
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.0f / l_tot;
    if (qrow >= L) return;
    float* op = (float*)a.o + rid.q0 + (size_t)qrow * a.qs.rs;
#pragma unroll
    for (int T = 0; T < TDV; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dv = 32 * T + 8 * i + 4 * hh;
            float4 v;
            v.x = o[T][4 * i] * inv;
            v.y = o[T][4 * i + 1] * inv;
            v.z = o[T][4 * i + 2] * inv;
            v.w = o[T][4 * i + 3] * inv;
            *reinterpret_cast<float4*>(op + dv) = v;
        }
}

// ---------------------------------------------------------------------------
// V -> V^T [heads][d][NT] for one segment (head = b * Hkv + h), 64-key tiles
// through LDS; columns from L to NT (the rest of the last block) are zero.
// With PERMUTE, key n of every 16-key chunk is stored at position
// (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1): key groups [0-3, 8-11, 4-7, 12-15].
// ---------------------------------------------------------------------------
template <typename T, bool PERMUTE, int D>
__global__ __launch_bounds__(256) void k_transpose_v(const T* __restrict__ v, TokStride vs, int Hkv,
                                                     T* __restrict__ vt, int L, int NT) {
    constexpr int TK = 64, VEC = 16 / (int)sizeof(T);   // elements per 16-byte access
    __shared__ __attribute__((aligned(16))) T tile[TK][D + VEC];
    const int head = blockIdx.y, n0 = blockIdx.x * TK, tid = threadIdx.x;
    const T* src = v + (size_t)(head / Hkv) * vs.bst + (size_t)(head % Hkv) * vs.hs;
    // 16-byte row pieces in, one row of the tile per key (zero past L)
    for (int e = tid; e < TK * D / VEC; e += 256) {
        const int n = e / (D / VEC), c = e % (D / VEC);
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (n0 + n < L) w = *reinterpret_cast<const uint4*>(src + (size_t)(n0 + n) * vs.rs + c * VEC);
        *reinterpret_cast<uint4*>(&tile[n][c * VEC]) = w;
    }
    __syncthreads();
    // 16-byte pieces out: VEC consecutive key positions of one V^T row
    T* dst = vt + (size_t)head * D * NT + n0;
    for (int e = tid; e < D * TK / VEC; e += 256) {
        const int dd = e / (TK / VEC), p0 = (e % (TK / VEC)) * VEC;
        union {
            uint4 w;
            T x[VEC];
        } u;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const int p = p0 + k;
            const int n = PERMUTE ? ((p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1)) : p;
            u.x[k] = tile[n][dd];
        }
        *reinterpret_cast<uint4*>(dst + (size_t)dd * NT + p0) = u.w;
    }
}

// Attention order of the heads: within each run of `group` consecutive heads
// (the query heads of one key/value head of one sequence) the heads sorted by
// their block count, most first, ties by index.  hperm[grp * group + rank] = head.
__global__ __launch_bounds__(64) void k_head_order(const unsigned long long* __restrict__ tot, int* __restrict__ hperm,
                                                   int group) {
    const int base = blockIdx.x * group;
    for (int g = threadIdx.x; g < group; g += 64) {
        const unsigned long long t = tot[base + g];
        int rank = 0;
        for (int j = 0; j < group; ++j) {
            const unsigned long long u = tot[base + j];
            rank += (u > t || (u == t && j < g)) ? 1 : 0;
        }
        hperm[base + rank] = base + g;
    }
}

hipError_t launch_head_order(const unsigned long long* total_blocks, int* hperm, int nheads, int group,
                             hipStream_t st) {
    if (nheads <= 0 || group <= 0 || nheads % group != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_head_order, dim3(nheads / group), dim3(64), 0, st, total_blocks, hperm, group);
    return hipGetLastError();
}

template <int D>
static void launch_transpose_v_t(const void* v, const TokStride& vs, void* vt, int dtype_bf16, int nseq, int Hkv,
                                 int L, int NT, hipStream_t st) {
    const dim3 g(NT / 64, nseq * Hkv);
    if (dtype_bf16)
        hipLaunchKernelGGL((k_transpose_v<bf16_t, true, D>), g, dim3(256), 0, st, (const bf16_t*)v, vs, Hkv,
                           (bf16_t*)vt, L, NT);
    else
        hipLaunchKernelGGL((k_transpose_v<float, false, D>), g, dim3(256), 0, st, (const float*)v, vs, Hkv,
                           (float*)vt, L, NT);
}

hipError_t launch_transpose_v(const void* v, const TokStride& vs, void* vt, int dtype_bf16, int d, int nseq, int Hkv,
                              int L, int NT, hipStream_t st) {
    if (d == 128) launch_transpose_v_t<128>(v, vs, vt, dtype_bf16, nseq, Hkv, L, NT, st);
    else if (d == 64) launch_transpose_v_t<64>(v, vs, vt, dtype_bf16, nseq, Hkv, L, NT, st);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <bool SPARSE, bool GATHER, int D>
static void launch_attention_t(const AttnArgs& a, hipStream_t st) {
    const unsigned items = (unsigned)a.items;
    if (a.dtype_bf16) {
        // Dense rows at block 128 also run in pairs (an eight-wave workgroup, one
        // per CU): 4-5 % faster than one row per workgroup there, while on the
        // sparse selections the pairs' list unions cost more than the shared
        // tile loads save.
        if (a.BS == 128 && !SPARSE)
            hipLaunchKernelGGL((k_attn_bf16<128, false, false, true, D>), dim3(items), dim3(512), 0, st, a);
        else if (a.BS == 128)
            hipLaunchKernelGGL((k_attn_bf16<128, SPARSE, GATHER, false, D>), dim3(items), dim3(256), 0, st, a);
        else
            hipLaunchKernelGGL((k_attn_bf16<64, SPARSE, GATHER, true, D>), dim3(items), dim3(256), 0, st, a);
    } else {
        const size_t lds = (size_t)2 * (kKT * (D + 4) + D * (kKT + 4)) * sizeof(float);
        if (a.BS == 128) {
            (void)hipFuncSetAttribute((const void*)k_attn_f32<128, SPARSE, GATHER, D>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            hipLaunchKernelGGL((k_attn_f32<128, SPARSE, GATHER, D>), dim3(items), dim3(256), lds, st, a);
        } else {
            (void)hipFuncSetAttribute((const void*)k_attn_f32<64, SPARSE, GATHER, D>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            hipLaunchKernelGGL((k_attn_f32<64, SPARSE, GATHER, D>), dim3(items), dim3(128), lds, st, a);
        }
    }
}

template <int D>
static void launch_attention_d(const AttnArgs& a, hipStream_t st) {
    if (!a.lists) launch_attention_t<false, false, D>(a, st);
    else if (a.colptr) launch_attention_t<true, true, D>(a, st);
    else launch_attention_t<true, false, D>(a, st);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
    // bf16 at block 64, and bf16 dense rows, run query-block pairs; the work
    // items must have been counted that way
    if (a.dtype_bf16 && (a.BS == 64 || !a.lists) && !a.pair) return hipErrorInvalidValue;
    if (a.d == 128) launch_attention_d<128>(a, st);
    else if (a.d == 64) launch_attention_d<64>(a, st);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Token-granular columns: per query head, the K rows of its selected columns
// (ascending) as Kg [NT][d] and their V values transposed as V^T [d][NT]
// (same 16-key permutation as the main V^T for bf16), zero past the last
// column of the 64-column tile.  grid (NT / 64, nseq * Hq); heads without
// columns return at once.
// ---------------------------------------------------------------------------
template <typename T, bool PERMUTE, int D>
__global__ __launch_bounds__(256) void k_gather_cols(const T* __restrict__ k, const T* __restrict__ v, TokStride ks,
                                                     int Hq, int Hkv, int L, int nb, int NT,
                                                     const int* __restrict__ colptr, const int* __restrict__ colidx,
                                                     T* __restrict__ kg, T* __restrict__ vgt) {
    constexpr int TK = 64;
    __shared__ T tile[TK][D + 2];
    __shared__ int js[TK];
    const int bh = blockIdx.y, c0 = blockIdx.x * TK, tid = threadIdx.x;
    const int ncol = colptr[(size_t)bh * (nb + 1) + nb];
    if (c0 >= ncol) return;
    const int b = bh / Hq, kvh = (bh % Hq) / (Hq / Hkv);
    const size_t base = (size_t)b * ks.bst + (size_t)kvh * ks.hs;
    if (tid < TK) js[tid] = c0 + tid < ncol ? colidx[(size_t)bh * L + c0 + tid] : -1;
    __syncthreads();
    T* kd = kg + ((size_t)bh * NT + c0) * D;
    for (int e = tid; e < TK * D; e += 256) {
        const int n = e / D, dd = e % D;
        const int j = js[n];
        kd[(size_t)n * D + dd] = j >= 0 ? k[base + (size_t)j * ks.rs + dd] : (T)0;
        tile[n][dd] = j >= 0 ? v[base + (size_t)j * ks.rs + dd] : (T)0;
    }
    __syncthreads();
    T* dst = vgt + (size_t)bh * D * NT + c0;
    for (int e = tid; e < TK * D; e += 256) {
        const int dd = e / TK, p = e % TK;
        const int n = PERMUTE ? ((p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1)) : p;
        dst[(size_t)dd * NT + p] = tile[n][dd];
    }
}

template <int D>
static void launch_gather_cols_t(const void* k, const void* v, const TokStride& ks, int dtype_bf16, int nseq, int Hq,
                                 int Hkv, int L, int nb, int NT, const int* colptr, const int* colidx, void* kg,
                                 void* vgt, hipStream_t st) {
    const dim3 g(NT / 64, nseq * Hq);
    if (dtype_bf16)
        hipLaunchKernelGGL((k_gather_cols<bf16_t, true, D>), g, dim3(256), 0, st, (const bf16_t*)k, (const bf16_t*)v,
                           ks, Hq, Hkv, L, nb, NT, colptr, colidx, (bf16_t*)kg, (bf16_t*)vgt);
    else
        hipLaunchKernelGGL((k_gather_cols<float, false, D>), g, dim3(256), 0, st, (const float*)k, (const float*)v,
                           ks, Hq, Hkv, L, nb, NT, colptr, colidx, (float*)kg, (float*)vgt);
}

hipError_t launch_gather_cols(const void* k, const void* v, const TokStride& ks, int dtype_bf16, int d, int nseq,
                              int Hq, int Hkv, int L, int nb, int NT, const int* colptr, const int* colidx, void* kg,
                              void* vgt, hipStream_t st) {
    if (d == 128) launch_gather_cols_t<128>(k, v, ks, dtype_bf16, nseq, Hq, Hkv, L, nb, NT, colptr, colidx, kg, vgt, st);
    else if (d == 64) launch_gather_cols_t<64>(k, v, ks, dtype_bf16, nseq, Hq, Hkv, L, nb, NT, colptr, colidx, kg, vgt, st);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace fp
