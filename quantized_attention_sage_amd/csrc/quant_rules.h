// Per-token quantization rules shared by the prologue and by the attention
// kernel's fused Q path, so that both produce the same codes bit for bit.
// Internal; included inside namespace sage { namespace { ... } }.
#pragma once

template <typename T>
__device__ __forceinline__ float to_f32(uint16_t bits);

template <>
__device__ __forceinline__ float to_f32<__half>(uint16_t bits) {
    return __half2float(__ushort_as_half(bits));
}

template <>
__device__ __forceinline__ float to_f32<__hip_bfloat16>(uint16_t bits) {
    return __uint_as_float(static_cast<uint32_t>(bits) << 16);
}

__device__ __forceinline__ int8_t int8_code(float x, float r) {
    float y = x * r;
    float n = rintf(y);
    n = fminf(fmaxf(n, -127.0f), 127.0f);
    return static_cast<int8_t>(static_cast<int>(n));
}

// Load 8 consecutive channels [d0, d0 + 8) of one token row; channels >= D
// read as 0. VEC: one 16-byte load (caller guarantees alignment and D % 8 == 0).
template <typename T, bool VEC>
__device__ __forceinline__ void load8(const uint16_t* row, int d0, int D, float (&x)[8]) {
    if (VEC) {
        if (d0 < D) {
            uint4 u = *reinterpret_cast<const uint4*>(row + d0);
            uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[2 * i] = to_f32<T>(static_cast<uint16_t>(w[i] & 0xFFFFu));
                x[2 * i + 1] = to_f32<T>(static_cast<uint16_t>(w[i] >> 16));
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.0f;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (d0 + i < D) ? to_f32<T>(row[d0 + i]) : 0.0f;
    }
}

