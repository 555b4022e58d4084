// bench_mfma_roof.hip -- the bf16 matrix-core rate this GPU sustains.
//
// Each wave issues iters x 16 v_mfma_f32_32x32x16_bf16 on register operands
// (eight independent accumulators), two waves per SIMD, and writes its
// accumulator sum once at the end; there is no other memory traffic.  Run
// with constant operands (0.5) and with pseudo-random ones (uniform in
// [-1, 1)): the matrix cores' power, and so the clock they sustain, depends on
// how many operand bits toggle.  Built and run by `python3 bench.py
// --mfma-roof`; prints TFLOP/s per run (the first runs of each kind ramp the
// clock up).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
void roof(const unsigned* __restrict__ seed, float* __restrict__ out, int iters, int randomize) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  unsigned x = seed[threadIdx.x] ^ (tid * 2654435761u);
  bf16x8 a[4], b[4];
  for (int i = 0; i < 4; i++)
    for (int j = 0; j < 8; j++) {
      x = x * 1664525u + 1013904223u;
      float v = randomize ? ((int)(x >> 16) - 32768) / 32768.0f : 0.5f;
      a[i][j] = (__bf16)v;
      x = x * 1664525u + 1013904223u;
      v = randomize ? ((int)(x >> 16) - 32768) / 32768.0f : 0.5f;
      b[i][j] = (__bf16)v;
    }
  f32x16 c[8];
  for (int i = 0; i < 8; i++) c[i] = f32x16{};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int k = 0; k < 2; k++)
#pragma unroll
      for (int i = 0; i < 8; i++) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + k) & 3], b[i & 3], c[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 8; i++)
    for (int j = 0; j < 16; j++) s += c[i][j];
  out[tid] = s;
}

int main(int argc, char** argv) {
  const int blocks = argc > 1 ? atoi(argv[1]) : 1024;
  const int iters = argc > 2 ? atoi(argv[2]) : 2000;
  unsigned* seed; float* out;
  if (hipMalloc(&seed, 512 * 4) != hipSuccess || hipMalloc(&out, (size_t)blocks * 512 * 4) != hipSuccess) {
    printf("allocation failed\n");
    return 1;
  }
  unsigned hs[512]; for (int i = 0; i < 512; i++) hs[i] = 12345u + 777u * i;
  if (hipMemcpy(seed, hs, sizeof hs, hipMemcpyHostToDevice) != hipSuccess) return 1;
  hipEvent_t e0, e1;
  (void)hipEventCreate(&e0);
  (void)hipEventCreate(&e1);
  for (int rnd = 0; rnd < 2; rnd++) {
    for (int r = 0; r < 5; r++) {  // warm-up then timed
      (void)hipEventRecord(e0);
      hipLaunchKernelGGL(roof, dim3(blocks), dim3(512), 0, 0, seed, out, iters, rnd);
      (void)hipEventRecord(e1);
      (void)hipEventSynchronize(e1);
      float ms = 0.f;
      (void)hipEventElapsedTime(&ms, e0, e1);
      double flops = (double)blocks * 8 * iters * 16 * 32768.0;
      printf("%s run %d: %.3f ms  %.1f TFLOP/s\n", rnd ? "random" : "constant", r, ms, flops / (ms * 1e-3) / 1e12);
    }
  }
  hipError_t e = hipGetLastError();
  printf("status %s\n", hipGetErrorString(e));
  return e != hipSuccess;
}
