// Internal interface between the host library and the kernel translation units.
#pragma once

#include "fp_common.h"

namespace fp {

constexpr int kHeadDim = 128;        // supported head dimension
constexpr int kMaxBlock = 128;       // largest supported block size
constexpr int kMaxBlocks = 4096;     // largest supported N / block
constexpr int kScoreDSConst = 32;    // d-slice of the last-block score kernel
constexpr int kRadixBits = 11;       // bits resolved per selection pass
constexpr int kRadixBins = 1 << kRadixBits;
constexpr int kSelChunk = 4096;      // list elements per selection workgroup
constexpr int kGammaShift = 24;      // G = rint(gamma * 2^24)
constexpr unsigned char kPatternQueryAware = 1;

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

// Device buffers of a plan (passed by value to kernels).
struct PlanDev {
    int BH, BS, N, nb;
    long long tri;               // nb (nb + 1) / 2
    int mode_all;                // gamma == 1: every causal block
    int floor_blocks;            // max(1, ceil(min_budget / BS))
    int cap_blocks;              // ceil(max_budget / BS), 0 = uncapped
    int qa_querywise;            // query-aware heads select row by row
    unsigned long long G;        // rint(gamma 2^24)
    unsigned char* pattern;      // [BH]
    double* djs;                 // [BH]
    float* qbar;                 // [BH][nb][d]
    float* kbar;                 // [B*Hkv][nb][d]
    float* rowmax;               // [BH][BS]
    float* rowsum;               // [BH][BS]
    float* colsum;               // [BH][N]
    float* diagsum;              // [BH][N]
    float* atrue;                // [BH][nb]
    float* ahat;                 // [BH][tri]
    SelState* sel;               // [2 BH]
    unsigned long long* hist;    // [2 BH][kRadixBins]
    unsigned char* colblk;       // [BH][nb]
    unsigned char* diagA;        // [BH][nb]
    unsigned char* diagB;        // [BH][nb]
    float* colmass;              // [BH][nb]  selected column mass per key block (cap only)
    float* diagmass;             // [BH][nb]  selected diagonal mass per block diagonal (cap only)
    int* lists;                  // [BH][tri]  row r's list at offset r (r + 1) / 2
    int* counts;                 // [BH][nb]
    unsigned long long* total_blocks;  // [BH] selected blocks per head
};

// Inputs and transient workspace of one planning call.
struct PlanArgs {
    const void* q;
    const void* k;
    int dtype_bf16;
    int B, Hq, Hkv;
    double tau;
    unsigned long long G;
    Canon canon;
    float* s2;        // [BH][BS][N] transient
    float* pmax;      // [BH][ceil(N/256)][BS] transient
    float* rz;        // [BH][BS] transient
};

struct AttnArgs {
    const void* q;
    const void* k;
    const void* vt;      // V transposed: [B*Hkv][d][N]
    void* o;
    int dtype_bf16;
    int B, Hq, Hkv, N, BS, nb;
    const int* lists;    // nullptr: dense causal
    const int* counts;
    long long tri;
    float scale_log2;    // log2(e) / sqrt(d)
};

hipError_t launch_plan(const PlanArgs& a, PlanDev& P, hipStream_t st);
hipError_t launch_probe_exp2(const float* x, float* y, long long n, const Canon& K, hipStream_t st);
hipError_t launch_probe_ln(const double* x, double* y, long long n, const Canon& K, hipStream_t st);
hipError_t launch_probe_sqrt(const double* x, double* y, long long n, hipStream_t st);
hipError_t launch_transpose_v(const void* v, void* vt, int dtype_bf16, int heads, int N, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

}  // namespace fp
