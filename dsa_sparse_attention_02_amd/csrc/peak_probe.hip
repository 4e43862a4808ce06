// Peak probes of one gfx950 GPU, for the roofline figures of the benchmark:
// streamed HBM read and copy bandwidth, bf16 MFMA 32x32x16 throughput, and LDS
// read bandwidth (16-byte and transposed 8-byte reads).  Prints one JSON object.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#define CHECK(x)                                                                         \
    do {                                                                                 \
        hipError_t e_ = (x);                                                             \
        if (e_ != hipSuccess) {                                                          \
            fprintf(stderr, "peak_probe: %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                                    \
        }                                                                                \
    } while (0)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// grid-stride 16-byte copy
__global__ __launch_bounds__(256) void copy16(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, size_t n)
{
    for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) dst[i] = src[i];
}

// grid-stride 16-byte non-temporal read (folded into one word so it is not removed)
__global__ __launch_bounds__(256) void read16_nt(const u32x4 *__restrict__ src, size_t n, uint32_t *out)
{
    u32x4 acc = {0, 0, 0, 0};
    for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        acc ^= __builtin_nontemporal_load(src + i);
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) out[blockIdx.x] = 1;
}

// four independent bf16 MFMA chains per wave
__global__ __launch_bounds__(512) void mfma_bf16(float *out, int iters)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)(lane + i);
        b[i] = (__bf16)(float)(lane - i);
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
    float s = 0;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    if (s == 1.2345f) out[blockIdx.x] = s;
}

// LDS reads: each wave reads 1 KB rows (16 bytes per lane, conflict free), or
// transposed 8-byte reads; 64 KB of LDS per block
template <bool TR>
__global__ __launch_bounds__(512) void lds_read(uint32_t *out, int iters)
{
    __shared__ u32x4 buf[4096];
    for (int i = threadIdx.x; i < 4096; i += 512) buf[i] = u32x4{(uint32_t)i, (uint32_t)i * 3u, 5u, 7u};
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    u32x4 acc = {0, 0, 0, 0};
    s16x4 acc2 = {0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if constexpr (TR) {
                const int off = (((wave * 16 + u + it) & 127) * 512) + lane * 8;
                acc2 ^= __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)((__attribute__((address_space(3))) char *)buf + off));
            } else {
                acc ^= buf[((wave * 16 + u + it) & 63) * 64 + lane];
            }
        }
    }
    const uint32_t t2 = ((uint32_t)(uint16_t)acc2[0] | ((uint32_t)(uint16_t)acc2[1] << 16)) ^
                        ((uint32_t)(uint16_t)acc2[2] | ((uint32_t)(uint16_t)acc2[3] << 16));
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w ^ t2) == 0x12345678u) out[blockIdx.x] = 1;
}

template <typename F>
static float time_ms(F f, int reps)
{
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0f;
    f();
    (void)hipDeviceSynchronize();
    (void)hipEventRecord(a);
    for (int i = 0; i < reps; ++i) f();
    (void)hipEventRecord(b);
    (void)hipEventSynchronize(b);
    float ms = -1.0f;
    (void)hipEventElapsedTime(&ms, a, b);
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    return ms / reps;
}

int main()
{
    int cus = 0, clk_khz = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    CHECK(hipDeviceGetAttribute(&clk_khz, hipDeviceAttributeClockRate, 0));
    uint32_t *o = nullptr;
    CHECK(hipMalloc(&o, 1 << 20));
    const size_t n = (size_t)1 << 26;  // 1 GiB of 16-byte elements
    u32x4 *src = nullptr, *dst = nullptr;
    CHECK(hipMalloc(&src, n * 16));
    CHECK(hipMalloc(&dst, n * 16));
    CHECK(hipMemset(src, 1, n * 16));
    double best_read = 0, best_copy = 0;
    for (int grid : {1024, 2048, 4096}) {
        const float rd = time_ms([&] { hipLaunchKernelGGL(read16_nt, dim3(grid), dim3(256), 0, 0, src, n, o); }, 10);
        const float cp = time_ms([&] { hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, 0, src, dst, n); }, 10);
        if (rd > 0 && n * 16 / (rd * 1e6) > best_read) best_read = n * 16 / (rd * 1e6);
        if (cp > 0 && 2.0 * n * 16 / (cp * 1e6) > best_copy) best_copy = 2.0 * n * 16 / (cp * 1e6);
    }
    const int mit = 20000;
    const float mm = time_ms([&] { hipLaunchKernelGGL(mfma_bf16, dim3(cus * 2), dim3(512), 0, 0, (float *)o, mit); }, 3);
    const double mfma_tflops = (double)cus * 2 * 8 * mit * 4 * 32768.0 / (mm * 1e9);
    const int lit = 4096, lgrid = cus * 4;
    const float l128 = time_ms([&] { hipLaunchKernelGGL(lds_read<false>, dim3(lgrid), dim3(512), 0, 0, o, lit); }, 5);
    const float ltr = time_ms([&] { hipLaunchKernelGGL(lds_read<true>, dim3(lgrid), dim3(512), 0, 0, o, lit); }, 5);
    const double clk = clk_khz * 1e3;
    const double b128 = (double)lgrid * 512 * lit * 16 * 16 / (l128 * 1e-3) / cus / clk;
    const double btr = (double)lgrid * 512 * lit * 16 * 8 / (ltr * 1e-3) / cus / clk;
    CHECK(hipDeviceSynchronize());
    printf("{\"cus\": %d, \"clock_mhz\": %.0f, \"hbm_read_nt_gbps\": %.1f, \"hbm_copy_gbps\": %.1f, "
           "\"mfma_bf16_tflops\": %.1f, \"lds_b128_bytes_per_clk_cu\": %.1f, \"lds_tr8_bytes_per_clk_cu\": %.1f}\n",
           cus, clk / 1e6, best_read, best_copy, mfma_tflops, b128, btr);
    CHECK(hipFree(src));
    CHECK(hipFree(dst));
    CHECK(hipFree(o));
    return 0;
}
