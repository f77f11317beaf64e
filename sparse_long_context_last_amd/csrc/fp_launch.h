// Internal interface between the host library and the kernel translation units.
#pragma once

#include "fp_common.h"

namespace fp {

constexpr int kMaxHeadDim = 128;     // supported head dimensions: 64 and 128
constexpr int kMaxBlock = 128;       // largest supported block size
constexpr int kMaxBlocks = 4096;     // largest supported N / block
constexpr int kScoreDSConst = 32;    // d-slice of the last-block score kernel
constexpr int kRadixBits = 11;       // bits resolved per selection pass
constexpr int kRadixBins = 1 << kRadixBits;
constexpr int kSelChunk = 4096;      // list elements per selection workgroup (twice that for long lists)
constexpr long long kSelLongList = 262144;
constexpr int kSelMaxPasses = 5;     // radix passes over 31 value bits + at most 24 index bits
constexpr int kSelHistBufs = 3;      // histogram buffers the passes rotate through
constexpr int kGammaShift = 24;      // G = rint(gamma * 2^24)
// the longest selection list (the causal triangle of kMaxBlocks rows) fits the pass buffers
static_assert(31 + index_bits((long long)kMaxBlocks * (kMaxBlocks + 1) / 2) <= kRadixBits * kSelMaxPasses,
              "selection passes");
constexpr unsigned char kPatternQueryAware = 1;
constexpr size_t kNoAllocScratchBytes = 64ull << 20;   // device workspace of fp_prefill_attend_noalloc

// State of one selection list (per head: slot 0 and slot 1).
struct SelState {
    unsigned long long U;       // total fixed-point mass
    unsigned long long T;       // threshold ceil(G U / 2^24)
    unsigned long long R;       // mass still to reach inside the current prefix
    unsigned long long prefix;  // resolved high key bits
    unsigned long long kstar;   // key of the last selected element (when has)
    int ibits;                  // index bits of the key
    int pos;                    // key bits still unresolved
    int active;                 // selection passes still running
    int has;                    // list selects at least one element
};

// Token addressing of a Q/O or K/V tensor inside one segment: element c of
// token t of head h of the segment's sequence b sits at
//   base + b * bst + h * hs + t * rs + c
// (base: the segment's first token, applied on the host).  [B, H, N, d]
// tensors have rs = d, hs = N d, bst = H N d; packed [T, H, d] tensors have
// rs = H d, hs = d and one sequence per segment.
struct TokStride {
    long long rs, hs, bst;
};

// Device buffers of one plan segment: heads that share one sequence length L
// (passed by value to kernels).  Every length L >= 1 is allowed; the last
// block of a sequence holds L - (nb - 1) BS tokens.
struct PlanDev {
    int BH, BS;
    int L;                       // tokens of every head of the segment
    int NS;                      // row stride of the last-block score workspace (multiple of 256, >= L)
    int nb;                      // ceil(L / BS)
    int tail;                    // query rows of the last block row, L - (nb - 1) BS
    long long tri;               // nb (nb + 1) / 2
    int mode_all;                // gamma == 1: every causal block
    int floor_blocks;            // max(1, ceil(min_budget / BS))
    int cap_blocks;              // ceil(max_budget / BS), 0 = uncapped
    int qa_querywise;            // query-aware heads select row by row
    int vs_token;                // vertical-slash columns attended token by token
    unsigned long long G;        // rint(gamma 2^24)
    unsigned char* pattern;      // [BH]
    double* djs;                 // [BH]
    float* qbar;                 // [BH][nb][d]
    float* kbar;                 // [sequences * Hkv][nb][d]
    float* rowmax;               // [BH][BS]
    float* rowsum;               // [BH][BS]
    float* colsum;               // [BH][L]
    float* diagsum;              // [BH][L]
    float* atrue;                // [BH][nb]  (block sums of colsum until the divergence kernel normalises them)
    float* ahat;                 // [BH][tri]
    SelState* sel;               // [2 BH]  final selection state per list
    SelState* selk;              // [kSelMaxPasses][2 BH]  state before each radix pass
    unsigned long long* hist;    // [kSelHistBufs][2 BH][kRadixBins]  mass histograms, rotating over the passes
    unsigned char* colblk;       // [BH][nb]
    unsigned char* diagA;        // [BH][nb]
    unsigned char* diagB;        // [BH][nb]
    unsigned char* diagT;        // [BH][nb]
    float* colmass;              // [BH][nb]  selected column mass per key block (cap only)
    float* diagmass;             // [BH][nb]  selected diagonal mass per block diagonal (cap only)
    int* colcount;               // [BH][nb]   selected columns per key block (token mode)
    int* colptr;                 // [BH][nb+1] exclusive prefix of colcount (token mode)
    int* colidx;                 // [BH][L]    selected columns ascending (token mode)
    int* lists;                  // [BH][tri]  row r's list at offset r (r + 1) / 2
    int* counts;                 // [BH][nb]
    unsigned long long* total_blocks;  // [BH] selected blocks per head
};

// Inputs and transient workspace of one segment's planning call.
struct PlanArgs {
    int d;            // head dimension (64 or 128)
    const void* q;    // the segment's first token of head 0 of its first sequence
    const void* k;
    TokStride qs, ks;
    int dtype_bf16;
    int nseq, Hq, Hkv;  // sequences in the segment (BH = nseq Hq)
    double tau;
    unsigned long long G;
    Canon canon;
    float* s2;        // [BH][BS][NS] transient
    float* pmax;      // [BH][NS/256][BS] transient
    float* rz;        // [BH][BS] transient
    float* qt;        // [BH][d][BS] transient: the last block's queries, fp32, transposed
    hipStream_t aux;  // second stream for the pooling kernels (nullptr: all on the call's stream)
};

// One segment of the attention work (device table, one entry per segment).
struct AttnSeg {
    long long item0;      // first work item (one per head and query block)
    long long qoff, koff; // element offsets of the segment base in Q/O and in K/V
    long long vtoff;      // element offset of the segment in the V^T workspace
    long long loff, coff; // offsets of the segment in the plan's lists and counts
    long long goff;       // element offset of the segment in the gathered-column K and V^T buffers
    long long cpoff, cioff; // offsets of the segment in colptr and colidx
    long long hoff;       // global index (sequence * Hq + head) of the segment's first head
    int nseq;             // sequences (query heads = nseq Hq)
    int L, nb, NT;        // tokens, blocks, V^T row length nb BS
    int npi;              // work items per head: nb, or (nb + 1) / 2 with two query blocks per item
};

static_assert(sizeof(AttnSeg) % 4 == 0, "segment tables are uploaded as 32-bit words");

struct AttnArgs {
    int d;               // head dimension (64 or 128)
    const void* q;
    const void* k;
    const void* vt;      // V transposed, per segment [nseq Hkv][d][NT], zero past L
    void* o;
    int dtype_bf16;
    int Hq, Hkv, BS;
    int pair;            // two query blocks per workgroup (bf16: block 64, and dense rows)
    TokStride qs, ks;
    const AttnSeg* segs; // device
    int nseg;
    long long items;
    const int* lists;    // nullptr: dense causal
    const int* counts;
    const int* hperm;    // sparse: global head order (heads of each kv group, most blocks first); nullptr: identity
    const int* colptr;   // token-granular columns (nullptr: none)
    const int* colidx;
    const void* kg;      // gathered K rows     per head [NT][d]
    const void* vgt;     // gathered V^T        per head [d][NT]
    float scale_log2;    // log2(e) / sqrt(d)
};

hipError_t launch_plan(const PlanArgs& a, PlanDev& P, hipStream_t st);
hipError_t launch_fill_u32(unsigned int* p, unsigned int v, long long n, hipStream_t st);
// Copies a host table (bytes a multiple of 4) to device memory in stream order.
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t st);
hipError_t launch_zero3_u32(unsigned int* a, long long na, unsigned int* b, long long nb, unsigned int* c,
                           long long nc, hipStream_t st);
hipError_t launch_probe_exp2(const float* x, float* y, long long n, const Canon& K, hipStream_t st);
hipError_t launch_probe_ln(const double* x, double* y, long long n, const Canon& K, hipStream_t st);
hipError_t launch_probe_sqrt(const double* x, double* y, long long n, hipStream_t st);
hipError_t launch_transpose_v(const void* v, const TokStride& vs, void* vt, int dtype_bf16, int d, int nseq, int Hkv,
                              int L, int NT, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);
// Device address and size of the allocation-free call's workspace on the
// current device (looked up once per device).
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
hipError_t launch_head_order(const unsigned long long* total_blocks, int* hperm, int nheads, int group,
                             hipStream_t st);
hipError_t launch_gather_cols(const void* k, const void* v, const TokStride& ks, int dtype_bf16, int d, int nseq,
                              int Hq, int Hkv, int L, int nb, int NT, const int* colptr, const int* colidx, void* kg,
                              void* vgt, hipStream_t st);

}  // namespace fp
