// Issue-rate probe for the numbers the scan kernels are designed around (gfx950):
//   * fp32 FMA and v_exp_f32 throughput per CU and clock, at 1-8 resident waves per SIMD;
//   * one scan token over 8 states with wave-uniform B/C (exp2, two multiplies, two FMAs);
//   * a multiply whose operand comes through DPP row_newbcast (cross-lane broadcast);
//   * a plain 1 GiB device copy (practical HBM ceiling).
// Every kernel reads only its scalar arguments and writes one float per launched thread to
// `out`, which holds one float per thread; the copy touches n elements with a grid-stride loop.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
      std::exit(1);                                                                   \
    }                                                                                 \
  } while (0)

template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + K, 0xf, 0xf, true));
}

enum { kFma = 0, kExp = 1, kToken = 2, kDppMul = 3, kKinds = 4 };

template <int KIND>
__global__ __launch_bounds__(256) void rate_kernel(float* out, int iters, float seed, float b0, float b1, float b2,
                                                   float b3, float b4, float b5, float b6, float b7) {
  const float t = seed * static_cast<float>(threadIdx.x + 1) * 1e-7f;
  float v[8], A2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = t * static_cast<float>(i + 1);
    A2[i] = -0.1f * static_cast<float>(i + 1) * seed;
  }
  const float c = t * 0.5f + 0.25f, x = t * 0.25f + 0.5f;
  float acc = 0.0f;
  for (int it = 0; it < iters; ++it) {
    if (KIND == kFma) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], c, x);
    } else if (KIND == kExp) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_amdgcn_exp2f(v[i]);
    } else if (KIND == kToken) {
      const float dl = x * 0.01f + 0.001f * static_cast<float>(it & 7), du = dl * c;
      const float Bs[8] = {b0, b1, b2, b3, b4, b5, b6, b7};
      float an[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) an[i] = __builtin_amdgcn_exp2f(dl * A2[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(Bs[i], du, v[i] * an[i]);
      float y0 = 0.0f, y1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        y0 = __builtin_fmaf(Bs[7 - i], v[i], y0);
        y1 = __builtin_fmaf(Bs[6 - i], v[i + 1], y1);
      }
      acc += y0 + y1;
    } else {
      v[0] *= row_bcast<0>(c);
      v[1] *= row_bcast<1>(c);
      v[2] *= row_bcast<2>(c);
      v[3] *= row_bcast<3>(c);
      v[4] *= row_bcast<4>(c);
      v[5] *= row_bcast<5>(c);
      v[6] *= row_bcast<6>(c);
      v[7] *= row_bcast<7>(c);
    }
  }
  float s = acc;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += v[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy_kernel(const float4* __restrict__ a, float4* __restrict__ b, size_t n) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    b[i] = a[i];
}

int main() {
  hipDeviceProp_t p;
  CHECK(hipGetDeviceProperties(&p, 0));
  const int cus = p.multiProcessorCount;
  const double clk = p.clockRate * 1e3;
  std::printf("device %s, %d CUs, clock %.0f MHz; rates in elements (lane operations or state updates) per CU per clock\n",
              p.gcnArchName, cus, clk / 1e6);
  const char* names[kKinds] = {"fp32 FMA (8 chains)", "v_exp_f32 (8 chains)", "scan token, 8 states, uniform B/C",
                               "fp32 mul with DPP row_newbcast operand"};
  const int iters = 4096;
  for (int wps : {1, 2, 3, 4, 8}) {  // 256-thread blocks: one wave per SIMD per block
    const int blocks = cus * wps;
    float* out;
    CHECK(hipMalloc(&out, sizeof(float) * blocks * 256));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    for (int k = 0; k < kKinds; ++k) {
      auto launch = [&]() {
        switch (k) {
          case kFma: rate_kernel<kFma><<<blocks, 256>>>(out, iters, 1.f, .1f, .2f, .3f, .4f, .5f, .6f, .7f, .8f); break;
          case kExp: rate_kernel<kExp><<<blocks, 256>>>(out, iters, 1.f, .1f, .2f, .3f, .4f, .5f, .6f, .7f, .8f); break;
          case kToken: rate_kernel<kToken><<<blocks, 256>>>(out, iters, 1.f, .1f, .2f, .3f, .4f, .5f, .6f, .7f, .8f); break;
          default: rate_kernel<kDppMul><<<blocks, 256>>>(out, iters, 1.f, .1f, .2f, .3f, .4f, .5f, .6f, .7f, .8f); break;
        }
      };
      launch();
      CHECK(hipGetLastError());
      CHECK(hipDeviceSynchronize());
      CHECK(hipEventRecord(e0));
      for (int r = 0; r < 5; ++r) launch();
      CHECK(hipEventRecord(e1));
      CHECK(hipEventSynchronize(e1));
      float ms;
      CHECK(hipEventElapsedTime(&ms, e0, e1));
      ms /= 5;
      const double elems = static_cast<double>(blocks) * 256 * iters * 8;
      std::printf("waves/SIMD %d  %-40s %8.3f ms  %6.2f per CU per clock\n", wps, names[k], ms,
                  elems / (ms * 1e-3) / cus / clk);
    }
    CHECK(hipFree(out));
  }
  const size_t bytes = size_t{1} << 30, n = bytes / 16;
  float4 *a, *b;
  CHECK(hipMalloc(&a, bytes));
  CHECK(hipMalloc(&b, bytes));
  CHECK(hipMemset(a, 0, bytes));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int grid : {cus * 8, cus * 32}) {
    copy_kernel<<<grid, 256>>>(a, b, n);
    CHECK(hipGetLastError());
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < 5; ++r) copy_kernel<<<grid, 256>>>(a, b, n);
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    ms /= 5;
    std::printf("copy 1 GiB, grid %d: %.3f ms, %.1f GB/s (read + write)\n", grid, ms, 2.0 * bytes / (ms * 1e-3) / 1e9);
  }
  CHECK(hipFree(a));
  CHECK(hipFree(b));
  return 0;
}
