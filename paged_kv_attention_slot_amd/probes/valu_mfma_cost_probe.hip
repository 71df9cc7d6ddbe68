// Issue cost of the softmax's vector instructions on gfx950, alone and beside
// v_mfma_f32_32x32x16_bf16: what bounds a prefill-chunk tile whose score
// weights (exp2 of a fused multiply-add, a bf16 pack, a row max, a row sum)
// are formed on the vector ALU between its matrix products.
//
// Every compute unit runs one or two 256-thread workgroups (one or two
// wavefronts per SIMD).  A wavefront repeats an iteration ITERS times:
//   * "alone": 8 groups of 8 vector instructions of one kind;
//   * "beside MFMA": 16 MFMAs over four independent accumulators, each
//     followed by NV vector instructions of one kind.
// The vector instructions work on 16 registers of their own, so none waits
// on an MFMA result.  A scheduling fence after each group keeps the order.
// The whole launch is timed with HIP events; the line gives nanoseconds per
// group per SIMD (the launch time over the groups one SIMD runs), so that
// "beside MFMA" minus "MFMA alone" is what the vector instructions add.
//
// Kinds: fma (v_fma_f32), exp (v_exp_f32), pack (v_cvt_pk_bf16_f32),
// max3 (v_maximum3_f32), dot2 (v_dot2_f32_bf16 against (1, 1)), and
// fma+exp (alternating), and exp_f16 (v_exp_f16, written in assembly).
// "(agpr)" lines: the same MFMAs written in assembly with their
// accumulators in AGPRs (the compiler's form keeps them in VGPRs); four
// s_nop 7 after the loop cover the last MFMA's result latency before the
// accumulators are read back.
//
// Build and run (one MI355X): `python -m paged_kv_attention_slot_amd.build
// --probe` writes _build/valu_mfma_cost_probe; run it with no arguments.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                 \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kIters = 512;
enum Kind { kFma, kExp, kPack, kMax3, kDot2, kFmaExp, kExp16 };
const char *const kNames[] = {"fma", "exp", "pack", "max3", "dot2", "fma+exp", "exp_f16"};

template <int K>
__device__ __forceinline__ void vop(float (&x)[16], int i, float c) {
  if constexpr (K == kFma) {
    x[i] = __builtin_fmaf(x[i], c, -0.5f);
  } else if constexpr (K == kExp) {
    x[i] = __builtin_amdgcn_exp2f(x[i]);
  } else if constexpr (K == kPack) {
    const bf16x2_t t = {static_cast<__bf16>(x[i]), static_cast<__bf16>(x[(i + 1) & 15])};
    x[i] = __builtin_bit_cast(float, t);
  } else if constexpr (K == kMax3) {
    x[i] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[i], x[(i + 5) & 15]), x[(i + 9) & 15]);
  } else if constexpr (K == kDot2) {
    const bf16x2_t one2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
    x[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x[(i + 3) & 15]), one2, x[i], false);
  } else if constexpr (K == kFmaExp) {
    x[i] = (i & 1) ? __builtin_amdgcn_exp2f(x[i]) : __builtin_fmaf(x[i], c, -0.5f);
  } else {
    float r;   // the half-precision exp2 on the low half of the register
    asm volatile("v_exp_f16 %0, %1" : "=v"(r) : "v"(x[i]));
    x[i] = r;
  }
}

// NM = 0: vector instructions alone (8 groups of NV); else NM MFMAs, each
// followed by NV vector instructions.  out holds one value per lane, so
// nothing is optimised away; it is never read.
template <int NM, int K, int NV, bool AG>
__global__ __launch_bounds__(256, 2) void cost_kernel(float *out, float seed) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(seed * (lane + i + 1) * 1e-3f);
    b[i] = static_cast<__bf16>(seed * (lane - i) * 1e-3f);
  }
  floatx16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = seed * 1e-3f * (lane + i);
  const float c = seed * 0.18f;
  for (int it = 0; it < kIters; ++it) {
    if constexpr (NM == 0) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
#pragma unroll
        for (int v = 0; v < NV; ++v) vop<K>(x, (g * NV + v) & 15, c);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if constexpr (AG)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[m & 3]) : "v"(a), "v"(b));
        else
          acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[m & 3], 0, 0, 0);
#pragma unroll
        for (int v = 0; v < NV; ++v) vop<K>(x, (m * NV + v) & 15, c);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if constexpr (AG) asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[j][i];
#pragma unroll
  for (int i = 0; i < 16; ++i) s += x[i];
  out[static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

template <int NM, int K, int NV, bool AG = false>
void run_case(int cus, float *out) {
  for (int per_simd = 1; per_simd <= 2; ++per_simd) {
    const int grid = cus * per_simd;   // out holds 2 * cus * 256 floats
    cost_kernel<NM, K, NV, AG><<<grid, 256>>>(out, 1.f);   // warm-up
    CHECK(hipGetLastError());
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    CHECK(hipEventRecord(e0, nullptr));
    cost_kernel<NM, K, NV, AG><<<grid, 256>>>(out, 1.f);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, nullptr));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    const int groups = NM == 0 ? 8 : NM;
    // one SIMD runs per_simd wavefronts of kIters x groups groups each
    const double ns = ms * 1e6 / (static_cast<double>(kIters) * groups * per_simd);
    if (NM == 0)
      std::printf("%d wave/SIMD  %-8s alone        8 per group : %6.2f ns per group per SIMD\n", per_simd,
                  kNames[K], ns);
    else
      std::printf("%d wave/SIMD  %-8s beside MFMA%s %d per MFMA  : %6.2f ns per MFMA per SIMD\n", per_simd,
                  NV ? kNames[K] : "(none)", AG ? "(agpr)" : "      ", NV, ns);
    std::fflush(stdout);
    CHECK(hipEventDestroy(e0));
    CHECK(hipEventDestroy(e1));
  }
}

int main() {
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  float *out = nullptr;
  CHECK(hipMalloc(&out, sizeof(float) * 2 * cus * 256));
  run_case<0, kFma, 8>(cus, out);
  run_case<0, kExp, 8>(cus, out);
  run_case<0, kPack, 8>(cus, out);
  run_case<0, kMax3, 8>(cus, out);
  run_case<0, kDot2, 8>(cus, out);
  run_case<0, kFmaExp, 8>(cus, out);
  run_case<0, kExp16, 8>(cus, out);
  run_case<16, kFma, 0>(cus, out);
  run_case<16, kFma, 4>(cus, out);
  run_case<16, kFma, 8>(cus, out);
  run_case<16, kExp, 2>(cus, out);
  run_case<16, kExp, 4>(cus, out);
  run_case<16, kExp, 8>(cus, out);
  run_case<16, kPack, 4>(cus, out);
  run_case<16, kMax3, 4>(cus, out);
  run_case<16, kDot2, 2>(cus, out);
  run_case<16, kDot2, 4>(cus, out);
  run_case<16, kFmaExp, 4>(cus, out);
  run_case<16, kFmaExp, 8>(cus, out);
  run_case<16, kExp16, 4>(cus, out);
  run_case<16, kFma, 0, true>(cus, out);
  run_case<16, kFma, 4, true>(cus, out);
  run_case<16, kFma, 8, true>(cus, out);
  run_case<16, kExp, 4, true>(cus, out);
  run_case<16, kFmaExp, 8, true>(cus, out);
  run_case<16, kPack, 4, true>(cus, out);
  run_case<16, kMax3, 4, true>(cus, out);
  run_case<16, kDot2, 4, true>(cus, out);
  CHECK(hipFree(out));
  std::printf("done\n");
  return 0;
}
