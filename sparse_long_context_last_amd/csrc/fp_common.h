// Shared device/host definitions of the gfx950 FlexPrefill library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp {

typedef uint16_t bf16_t;   // storage type of bfloat16 tensors

// Constants of the canonical selection arithmetic (computed on the host,
// passed by value to the kernels that need them).
struct Canon {
    float e2[8];       // 2^f Taylor coefficients: fp32 nearest to (ln 2)^k / k!
    double lnc[11];    // artanh series coefficients 1 / (2k + 1)
    double ln2;        // binary64 nearest to ln 2
    double sqrt_half;  // binary64 nearest to sqrt(1/2)
    float C;           // score scale log2(e) / sqrt(d), rounded once to fp32
};

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
    return __uint_as_float(((uint32_t)x) << 16);
}

template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) {
    return bf16_to_f32(*p);
}

// Round-to-nearest-even fp32 -> bf16 (inputs here are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

// Number of bits needed to write every index in [0, n).
__host__ __device__ constexpr int index_bits(long long n) {
    int b = 1;
    while ((1LL << b) < n) ++b;
    return b;
}

}  // namespace fp
