// Measurement program (not part of either library): what MI355X sustains for the
// per-logit instruction mix of the one-pass score kernel, with nothing else in the way.
//
// At d = 128 a wave of the score kernel issues, per 32x32x16 bf16 MFMA, two v_exp_f32
// and about four plain fp32 VALU instructions (one scale-and-reference fma and one add
// per logit, two logits per lane per MFMA).  Each mode below runs register-only loops
// of one such mix on every CU, 8 waves per CU (two per SIMD, as the score kernel), and
// prints the duration; with rocprofv3 counters (GRBM_GUI_ACTIVE for the clock,
// SQ_VALU_MFMA_BUSY_CYCLES for the matrix pipe) it gives the sustained clock and
// matrix rate of each mix.  Each thread writes one float of a buffer of
// CUs * 512 floats at the end; nothing else touches global memory.
//
// The LDS-fed modes read each MFMA's key operand from LDS as the score kernel does
// (one 16-byte read per lane, 1 KiB per wave, conflict-free): one read per MFMA is a
// wave holding one 32-row query tile (d = 256), one read per two MFMAs a wave holding
// two tiles that share the key operand (d = 128).  Per MFMA, d = 128 has two logits
// per lane (two exps, four fp32 instructions), d = 256 one (one exp, two).
//
//   block_wise_token_amd/probe_mfma_mix      (built by python -m block_wise_token_amd.build)
#include <hip/hip_runtime.h>

#include <cstdio>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define MFMA(acc, a, b) \
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define EXP(x) asm volatile("v_exp_f32 %0, %0" : "+v"(x))
#define FMA(x, y) asm volatile("v_fma_f32 %0, %0, %1, %1" : "+v"(x) : "v"(y))

// MODE 0: two independent MFMA chains, fixed operands.
// MODE 1: v_exp_f32 only.       MODE 2: v_fma_f32 only.
// MODE 3: per MFMA, E exps and F fmas from the same wave.
// MODE 4: waves 0-3 MFMA only, waves 4-7 the exps and fmas (work split across waves).
// MODE 5: two MFMA chains with an operand changed every step.
// MODE 6: as MODE 5 with both MFMAs of a step in one dependent chain.
template <int MODE, int E, int F>
__global__ __launch_bounds__(512, 1) void mix_kernel(float* out, int iters) {
  f32x16 acc0 = {}, acc1 = {};
  bf16x8 a, b;
  {
    uint32_t st = 2463534242u * (threadIdx.x + 1) + blockIdx.x * 977u;   // xorshift seeds
    for (int i = 0; i < 8; ++i) {
      st ^= st << 13;
      st ^= st >> 17;
      st ^= st << 5;
      a[i] = (__bf16)((float)(int)(st & 0xFFFF) * 3e-5f - 1.0f);
      st ^= st << 13;
      st ^= st >> 17;
      st ^= st << 5;
      b[i] = (__bf16)((float)(int)(st & 0xFFFF) * 3e-5f - 1.0f);
    }
  }
  float x[8], y = 1e-3f * threadIdx.x;
  for (int i = 0; i < 8; ++i) x[i] = -1.0f - 0.01f * i - 1e-4f * threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (MODE == 0) {
        MFMA(acc0, a, b);
        MFMA(acc1, a, b);
      }
      if (MODE == 5) {
        MFMA(acc0, a, b);
        MFMA(acc1, b, a);
        asm volatile("v_xor_b32 %0, %0, %1" : "+v"(a[0]) : "v"(y));
      }
      if (MODE == 6) {
        MFMA(acc0, a, b);
        MFMA(acc0, b, a);
        asm volatile("v_xor_b32 %0, %0, %1" : "+v"(a[0]) : "v"(y));
      }
      if (MODE == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) EXP(x[e]);
      }
      if (MODE == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) FMA(x[e], y);
      }
      if (MODE == 3) {
        MFMA(acc0, a, b);
#pragma unroll
        for (int e = 0; e < E; ++e) EXP(x[e & 7]);
#pragma unroll
        for (int f = 0; f < F; ++f) FMA(x[(f + 3) & 7], y);
        MFMA(acc1, a, b);
#pragma unroll
        for (int e = 0; e < E; ++e) EXP(x[(e + 4) & 7]);
#pragma unroll
        for (int f = 0; f < F; ++f) FMA(x[(f + 1) & 7], y);
      }
      if (MODE == 4) {
        if (wave < 4) {
          MFMA(acc0, a, b);
          MFMA(acc1, a, b);
        } else {
#pragma unroll
          for (int e = 0; e < 2 * E; ++e) EXP(x[e & 7]);
#pragma unroll
          for (int f = 0; f < 2 * F; ++f) FMA(x[(f + 3) & 7], y);
        }
      }
    }
  }
  float s = y;
  for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i];
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;   // grid = CUs x 512 threads
}

// LDS-fed mixes.  SHARE = 1: one key read per MFMA (a wave holding one query tile);
// SHARE = 2: one key read per two MFMAs (two tiles sharing the key operand).  CHAINS = 1
// accumulates every MFMA of a wave into one tile (one dependent chain, as one query
// tile over the whole head dimension does), CHAINS = 2 alternates two tiles.  The keys
// of an iteration's 16 MFMAs are requested one iteration ahead, as the score kernel
// requests a half-step's operands while it works on the previous one.  iters is even.
constexpr int kLdsKeys = 2048;   // 16-byte entries: 32 KiB of LDS
template <int SHARE, int E, int F, int CHAINS = 2>
__global__ __launch_bounds__(512, 1) void lds_mix_kernel(float* out, int iters) {
  constexpr int NR = 16 / SHARE;   // key reads per iteration
  __shared__ bf16x8 kbuf[kLdsKeys];
  f32x16 acc0 = {}, acc1 = {};
  bf16x8 a, b;
  {
    uint32_t st = 2463534242u * (threadIdx.x + 1) + blockIdx.x * 977u;   // xorshift seeds
    for (int i = 0; i < 8; ++i) {
      st ^= st << 13;
      st ^= st >> 17;
      st ^= st << 5;
      a[i] = (__bf16)((float)(int)(st & 0xFFFF) * 3e-5f - 1.0f);
      st ^= st << 13;
      st ^= st >> 17;
      st ^= st << 5;
      b[i] = (__bf16)((float)(int)(st & 0xFFFF) * 3e-5f - 1.0f);
    }
  }
  float x[8], y = 1e-3f * threadIdx.x;
  for (int i = 0; i < 8; ++i) x[i] = -1.0f - 0.01f * i - 1e-4f * threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // The block's threads fill the 2048 entries (blockDim.x divides 2048); every read
  // index is taken mod 2048.
  for (int j = threadIdx.x; j < kLdsKeys; j += blockDim.x) {
    bf16x8 v = a;
    v[j & 7] = b[(j >> 3) & 7];
    kbuf[j] = v;
  }
  __syncthreads();
  // Read r of iteration it: each wave reads 64 consecutive entries (1 KiB); the
  // addresses repeat every two iterations, so they are immediate offsets as in the
  // score kernel.
  auto fetch = [&](int it, bf16x8 (&kk)[NR]) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
      kk[r] = kbuf[(lane + 64 * (it * 16 + r) + 256 * wave) & (kLdsKeys - 1)];
  };
  auto body = [&](const bf16x8 (&kk)[NR]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      MFMA(acc0, kk[SHARE == 1 ? 2 * k : k], b);
#pragma unroll
      for (int e = 0; e < E; ++e) EXP(x[e & 7]);
#pragma unroll
      for (int f = 0; f < F; ++f) FMA(x[(f + 3) & 7], y);
      if (SHARE == 1 && CHAINS == 1) MFMA(acc0, kk[2 * k + 1], b);
      else if (SHARE == 1) MFMA(acc1, kk[2 * k + 1], b);
      else MFMA(acc1, kk[k], a);
#pragma unroll
      for (int e = 0; e < E; ++e) EXP(x[(e + 4) & 7]);
#pragma unroll
      for (int f = 0; f < F; ++f) FMA(x[(f + 1) & 7], y);
    }
  };
  bf16x8 k0[NR], k1[NR];
  fetch(0, k0);
  for (int it = 0; it < iters; it += 2) {
    fetch(it + 1, k1);
    body(k0);
    fetch(it + 2, k0);
    body(k1);
  }
  float s = y;
  for (int i = 0; i < 16; ++i) s += acc0[i] + acc1[i];
  for (int i = 0; i < 8; ++i) s += x[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;   // grid = CUs x (256 or 512) threads
}

static int run_kernel(void (*kern)(float*, int), const char* name, float* out, int cus,
                      int mfma_per_cu_iter, int threads = 512) {
  constexpr int kIters = 2000;
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 1;
  hipLaunchKernelGGL(kern, dim3(cus), dim3(threads), 0, 0, out, 10);
  if (hipDeviceSynchronize() != hipSuccess) return 1;
  (void)hipEventRecord(a);
  hipLaunchKernelGGL(kern, dim3(cus), dim3(threads), 0, 0, out, kIters);
  (void)hipEventRecord(b);
  if (hipEventSynchronize(b) != hipSuccess) return 1;
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  // an MFMA 32x32x16 is 32768 flops
  const double flops = (double)cus * kIters * mfma_per_cu_iter * 32768.0;
  std::printf("%-40s %9.1f us  %7.3f PFLOP/s of MFMA\n", name, ms * 1e3,
              flops / (ms * 1e-3) / 1e15);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return 0;
}

template <int MODE, int E, int F>
static int run(const char* name, float* out, int cus, int mfma_per_cu_iter) {
  return run_kernel(mix_kernel<MODE, E, F>, name, out, cus, mfma_per_cu_iter);
}
template <int SHARE, int E, int F, int CHAINS = 2>
static int run_lds(const char* name, float* out, int cus, int waves = 8) {
  return run_kernel(lds_mix_kernel<SHARE, E, F, CHAINS>, name, out, cus, 16 * waves, 64 * waves);
}

int main() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    std::printf("no device\n");
    return 1;
  }
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)cus * 512 * sizeof(float)) != hipSuccess) return 1;
  std::printf("%d CUs, 8 waves per CU (4 where marked), 2000 iterations of 8 steps per launch\n", cus);
  int bad = 0;
  // MFMAs per CU per iteration: 8 steps x 2 per wave, 8 waves (4 in the split mode)
  bad |= run<0, 0, 0>("mfma only (2 chains)", out, cus, 128);
  bad |= run<5, 0, 0>("mfma only, operand changing each step", out, cus, 128);
  bad |= run<1, 0, 0>("exp only", out, cus, 0);
  bad |= run<2, 0, 0>("fma only", out, cus, 0);
  bad |= run<3, 2, 0>("mfma + 2 exp each", out, cus, 128);
  bad |= run<3, 0, 4>("mfma + 4 fma each", out, cus, 128);
  bad |= run<3, 2, 4>("mfma + 2 exp + 4 fma each", out, cus, 128);
  bad |= run<4, 2, 4>("split: 4 mfma waves, 4 exp+fma waves", out, cus, 64);
  bad |= run<3, 1, 2>("mfma + 1 exp + 2 fma each", out, cus, 128);
  bad |= run_lds<1, 0, 0>("lds: one key read per mfma", out, cus);
  bad |= run_lds<1, 1, 2>("lds: one read per mfma + 1 exp + 2 fma", out, cus);
  bad |= run_lds<2, 0, 0>("lds: one key read per 2 mfma", out, cus);
  bad |= run_lds<2, 1, 2>("lds: one read per 2 mfma + 1 exp + 2 fma", out, cus);
  bad |= run_lds<2, 2, 4>("lds: one read per 2 mfma + 2 exp + 4 fma", out, cus);
  bad |= run<6, 0, 0>("mfma only, one chain, operand changing", out, cus, 128);
  bad |= run_lds<1, 1, 2, 1>("lds: one read per mfma + 1 exp + 2 fma, one chain", out, cus);
  // One wave per SIMD (4 waves per CU): a wave holding two 32-row tiles at d = 256
  bad |= run_lds<2, 1, 2>("4 waves: lds one read per 2 mfma + 1 exp + 2 fma", out, cus, 4);
  bad |= run_lds<1, 1, 2>("4 waves: lds one read per mfma + 1 exp + 2 fma", out, cus, 4);
  bad |= run_lds<2, 2, 4>("4 waves: lds one read per 2 mfma + 2 exp + 4 fma", out, cus, 4);
  (void)hipFree(out);
  return bad;
}
