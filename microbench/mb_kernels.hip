// Microbenchmarks of the gfx950 (MI355X, CDNA4) units the attention kernels
// are bound by, and a single-instruction accuracy probe of the matrix cores.
//
// They answer the questions the kernel design depends on:
//   * issue rate of the transcendental v_exp_f32 against v_fma_f32 / v_add_f32
//     (whether a software exp2 on the FMA path, as "FlashAttention 4: Atenção
//     Mais Rápida e Eficiente em Memória para LLMs", section "Exponenciais de
//     Software via Núcleos CUDA", proposes for the GPU it names, would
//     relieve a bottleneck here);
//   * the dense MFMA rate with accumulators in VGPRs or AGPRs, alone and
//     beside a softmax-like vector wave on the same SIMD (the overlap the
//     kernels rely on; "FlashAttention-3 ...", section "Interleaving de GEMM
//     e Softmax");
//   * LDS read bandwidth per compute unit for the read shapes the kernels
//     use (ds_read_b128, ds_read_b64, the transposing ds_read_b64_tr_b16),
//     and the MFMA rate when one operand streams from LDS;
//   * the error of one e4m3 / bf16 MFMA against the exact dot product.
//
// Every timed kernel records, per wave, the shader-clock counter
// (s_memtime) and the 100 MHz real-time counter (s_memrealtime) around its
// loop; rates are reported in cycles of the shader clock, so they do not
// depend on the clock the chip holds.  All accesses are in bounds by
// construction (LDS offsets are masked to the array; global buffers are
// indexed by block and wave only); every loop has a fixed trip count.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define MB_LDS __attribute__((address_space(3)))

// Per-wave record: shader clock at start and end, real-time clock at start
// and end, the wave's HW_ID register (SIMD, CU, shader array and engine
// fields) and XCC_ID (8 x uint64).  Written by lane 0 of each wave with a
// vector store.
struct Stamp {
  unsigned long long c0, c1, r0, r1, hw_id, xcc_id, pad0, pad1;
};

__device__ __forceinline__ void stamp_store(Stamp* out, int waves, unsigned long long c0,
                                            unsigned long long c1, unsigned long long r0,
                                            unsigned long long r1) {
  const int wave = threadIdx.x >> 6;
  unsigned hw, xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  if ((threadIdx.x & 63) == 0) {
    Stamp s = {c0, c1, r0, r1, hw, xcc, 0, 0};
    out[blockIdx.x * waves + wave] = s;
  }
}

// Occupancy guard: a timed kernel reserves PAD bytes of LDS (more than half
// of the 160 KiB of a compute unit) so that no two of its work-groups share
// a compute unit.  The array is touched only on a path no launch takes
// (iters < 0 is rejected by the host entry points), which keeps it
// allocated.
constexpr int PAD = 96 * 1024;
#define MB_RESERVE_LDS(iters)                                             \
  __shared__ unsigned char mb_pad[PAD];                                   \
  if ((iters) < 0) {                                                      \
    mb_pad[threadIdx.x] = (unsigned char)threadIdx.x;                     \
    __syncthreads();                                                      \
    sink[threadIdx.x] = (float)mb_pad[(threadIdx.x + 1) % blockDim.x];    \
    return;                                                               \
  }

// ---------------------------------------------------------------------------
// 1. vector ALU issue rate: 16 independent chains of one operation
// ---------------------------------------------------------------------------
// OP 0 v_fma_f32, 1 v_exp_f32, 2 v_add_f32, 3 v_cvt_pk_bf16_f32,
//    5 v_exp_f32 and v_fma_f32 alternating on independent chains (8 + 8),
//    4 a softmax mix: per pair of scores 2 fma, 2 exp, 2 add, 1 cvt_pk and
//      1 xor (which keeps the conversion live), 7 pairs per iteration.
// Vector instructions per iteration: 16 (OP 0-2, 5), 8 (OP 3), 57 (OP 4:
// the 7 x 8 above and one multiply).
template <int OP>
__global__ __launch_bounds__(1024, 1) void valu_rate(Stamp* out, float* sink, int iters,
                                                     float seed) {
  MB_RESERVE_LDS(iters);
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = seed * (float)(threadIdx.x + 3 * i + 1);
  const float a = seed * 0.5f, bconst = seed * 0.25f;
  unsigned pk = 0;
  __syncthreads();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (OP == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = __builtin_fmaf(x[i], a, bconst);
    } else if constexpr (OP == 1) {
      // 2^-x stays in (0.5, 1) from any start in (0, 1): no special values
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
    } else if constexpr (OP == 2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = x[i] + a;
    } else if constexpr (OP == 5) {
      // 8 exponential chains and 8 fma chains, independent of each other:
      // does the transcendental unit run beside the fma path?
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = __builtin_amdgcn_exp2f(-x[i]);
        x[i + 8] = __builtin_fmaf(x[i + 8], a, bconst);
      }
    } else if constexpr (OP == 3) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const f32x2 v = {x[i], x[i + 1]};
        // fed back as the next input, so every conversion stays live
        x[i] = __builtin_bit_cast(float, __builtin_convertvector(v, bf16x2));
      }
    } else {
      // the offset m depends on the previous iteration's sum, so nothing
      // is hoisted out of the loop
      const float m = x[14] * 1e-30f;
      float l0 = x[14], l1 = x[15];
#pragma unroll
      for (int i = 0; i < 14; i += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], a, m));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 1], a, m));
        const f32x2 v = {e0, e1};
        pk ^= __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
        l0 += e0;
        l1 += e1;
      }
      x[14] = l0;
      x[15] = l1;
    }
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float r = (float)pk;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += x[i];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
  stamp_store(out, blockDim.x >> 6, c0, c1, r0, r1);
}

// ---------------------------------------------------------------------------
// 2. MFMA rate, and MFMA beside a vector wave on the same SIMD
// ---------------------------------------------------------------------------
// Waves w < mfma_waves issue v_mfma_f32_32x32x16_bf16 on 4 independent
// accumulators (32 MFMAs per iteration); with `valu` set, waves 4-7 (those
// not issuing MFMAs) run the softmax mix of valu_rate<4> (57 vector
// instructions per mix iteration, 2 mix iterations per MFMA iteration: 114
// per 32 MFMAs, the attention kernels' ratio for 64 keys x 32 queries).  ACC 0: the
// accumulators in VGPRs (compiler builtin), ACC 1: in AGPRs (asm).
// Waves i and i + 4 of a work-group share a SIMD.
template <int ACC>
__global__ __launch_bounds__(512, 1) void mfma_pair(Stamp* out, float* sink, int iters,
                                                    int mfma_waves, int valu, float seed) {
  MB_RESERVE_LDS(iters);
  const int wave = threadIdx.x >> 6;
  float r = 0.f;
  __syncthreads();
  unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  if (wave < mfma_waves) {
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
      b[i] = (__bf16)(seed - (float)i);
    }
    f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if constexpr (ACC == 0) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc2, 0, 0, 0);
          acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc3, 0, 0, 0);
        } else {
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc0) : "v"(a), "v"(b));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc1) : "v"(a), "v"(b));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc2) : "v"(a), "v"(b));
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc3) : "v"(a), "v"(b));
        }
      }
    }
    if constexpr (ACC == 1) {
      // the asm MFMAs' results are read below; let the last ones retire
      asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
    }
    r = acc0[0] + acc1[1] + acc2[2] + acc3[3];
  } else if (valu && wave >= 4) {
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = seed * (float)(threadIdx.x + i);
    float l0 = 0.f, l1 = 0.f;
    unsigned pk = 0;
    const float cc = seed * 0.5f;
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < 2 * iters; ++it) {
      const float m = l0 * 1e-30f;
#pragma unroll
      for (int i = 0; i < 14; i += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cc, m));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i + 1], cc, m));
        const f32x2 v = {e0, e1};
        pk ^= __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
        l0 += e0;
        l1 += e1;
      }
    }
    r = l0 + l1 + (float)pk;
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
  stamp_store(out, 8, c0, c1, r0, r1);
}

// ---------------------------------------------------------------------------
// 3. LDS read bandwidth
// ---------------------------------------------------------------------------
// Every wave of the work-group reads a 64 KiB LDS array, 8 reads per
// iteration, consecutive lanes at consecutive addresses (no bank
// conflicts).  KIND 0 ds_read_b128 (1 KiB per wave instruction), 1
// ds_read_b64 (512 B), 2 ds_read_b64_tr_b16 (512 B; each 16-lane group
// reads 4 rows x 4 columns of 16-bit elements and transposes them).  The
// reads are written as one asm block per iteration that also waits for
// them (so no result register is live while its load is in flight); an
// empty asm consumes the results, so the loop carries no vector ALU work
// beyond one address add.  Offsets: the block's base address plus
// immediate offsets j * step, j < 8, with the base a multiple of 8 * step
// below 64 KiB, so every read stays inside the array.
#define MB_R128(j) "ds_read_b128 %" #j ", %8 offset:" #j "*1024\n\t"
#define MB_R64(op, j) #op " %" #j ", %8 offset:" #j "*512\n\t"
template <int KIND>
__global__ __launch_bounds__(1024, 1) void lds_read(Stamp* out, float* sink, int iters) {
  // 96 KiB, of which the reads cover the first 64: one work-group per CU
  constexpr int BYTES = 65536;
  constexpr int ALLOC = 96 * 1024;
  constexpr int STEP = KIND == 0 ? 1024 : 512;
  __shared__ __attribute__((aligned(16))) unsigned char lds[ALLOC];
  for (int i = threadIdx.x * 16; i < ALLOC; i += blockDim.x * 16)
    *(u32x4*)(lds + i) = u32x4{(unsigned)i, (unsigned)i + 1, (unsigned)i + 2, (unsigned)i + 3};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const unsigned lds0 = (unsigned)(size_t)((MB_LDS unsigned char*)lds);
  const unsigned base = lds0 + (unsigned)(lane * (STEP / 64));
  unsigned off = (unsigned)(wave * 8 * STEP) & (BYTES - 1);
  __syncthreads();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    const unsigned a = base + off;
    if constexpr (KIND == 0) {
      u32x4 v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile(MB_R128(0) MB_R128(1) MB_R128(2) MB_R128(3) MB_R128(4) MB_R128(5) MB_R128(6)
                   MB_R128(7) "s_waitcnt lgkmcnt(0)"
                   : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6),
                     "=&v"(v7)
                   : "v"(a)
                   : "memory");
      asm volatile("" ::"v"(v0), "v"(v1), "v"(v2), "v"(v3), "v"(v4), "v"(v5), "v"(v6), "v"(v7));
    } else if constexpr (KIND == 1) {
      u32x2 v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile(MB_R64(ds_read_b64, 0) MB_R64(ds_read_b64, 1) MB_R64(ds_read_b64, 2)
                   MB_R64(ds_read_b64, 3) MB_R64(ds_read_b64, 4) MB_R64(ds_read_b64, 5)
                   MB_R64(ds_read_b64, 6) MB_R64(ds_read_b64, 7) "s_waitcnt lgkmcnt(0)"
                   : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6),
                     "=&v"(v7)
                   : "v"(a)
                   : "memory");
      asm volatile("" ::"v"(v0), "v"(v1), "v"(v2), "v"(v3), "v"(v4), "v"(v5), "v"(v6), "v"(v7));
    } else {
      u32x2 v0, v1, v2, v3, v4, v5, v6, v7;
      asm volatile(MB_R64(ds_read_b64_tr_b16, 0) MB_R64(ds_read_b64_tr_b16, 1)
                   MB_R64(ds_read_b64_tr_b16, 2) MB_R64(ds_read_b64_tr_b16, 3)
                   MB_R64(ds_read_b64_tr_b16, 4) MB_R64(ds_read_b64_tr_b16, 5)
                   MB_R64(ds_read_b64_tr_b16, 6) MB_R64(ds_read_b64_tr_b16, 7)
                   "s_waitcnt lgkmcnt(0)"
                   : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3), "=&v"(v4), "=&v"(v5), "=&v"(v6),
                     "=&v"(v7)
                   : "v"(a)
                   : "memory");
      asm volatile("" ::"v"(v0), "v"(v1), "v"(v2), "v"(v3), "v"(v4), "v"(v5), "v"(v6), "v"(v7));
    }
    off = (off + 8 * STEP) & (BYTES - 1);
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = 0.f;
  stamp_store(out, blockDim.x >> 6, c0, c1, r0, r1);
}
#undef MB_R128
#undef MB_R64

// ---------------------------------------------------------------------------
// 4. MFMA with the A operand streamed from LDS (the kernels' matrix-core
//    phase: one 1 KiB ds_read_b128 fragment per 32x32x16 MFMA), optionally
//    beside a vector wave on each SIMD
// ---------------------------------------------------------------------------
// Waves w < mfma_waves read fragments of a 32 KiB LDS tile in the forward
// kernel's K-operand pattern (row = lane % 32, 16-byte chunk = 2 ks + lane/32,
// XOR-swizzled by the row) and issue one MFMA per fragment on 2 accumulators
// (the S^T product of one 64-key tile is 16 such MFMAs).  With `valu`, the
// other waves run the softmax mix as in mfma_pair.
__global__ __launch_bounds__(512, 1) void mfma_lds(Stamp* out, float* sink, int iters,
                                                   int mfma_waves, int valu, float seed) {
  constexpr int D = 128;
  // 32 KiB of K tiles, allocated as 96 KiB so that one work-group holds a CU
  __shared__ __attribute__((aligned(16))) __bf16 tile[64 * D * 2 * 3];
  for (int i = threadIdx.x; i < 64 * D * 2; i += blockDim.x) tile[i] = (__bf16)(seed * (float)i);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ln = lane & 31, lh = lane >> 5;
  float r = 0.f;
  unsigned long long c0 = __builtin_amdgcn_s_memtime();
  unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  if (wave < mfma_waves) {
    bf16x8 qf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[ks][i] = (__bf16)(seed * (float)(lane + ks + i));
    int koff[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) koff[ks] = ln * D + (((2 * ks + lh) ^ (ln & 15)) * 8);
    f32x16 s0 = {}, s1 = {};
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    // two tiles per iteration, so that each tile's address is a constant
    // folded into the reads' offsets
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const __bf16* kt = tile + t * 64 * D;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 a0 = *(const bf16x8*)(kt + koff[ks]);
          const bf16x8 a1 = *(const bf16x8*)(kt + 32 * D + koff[ks]);
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
    r = s0[0] + s1[5];
  } else if (valu && wave >= 4) {
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = seed * (float)(threadIdx.x + i);
    float l0 = 0.f, l1 = 0.f;
    unsigned pk = 0;
    const float cc = seed * 0.5f;
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    // 16 MFMAs per MFMA-wave iteration: 1 mix iteration (57 VALU), the
    // attention kernels' ratio
    for (int it = 0; it < iters; ++it) {
      const float m = l0 * 1e-30f;
#pragma unroll
      for (int i = 0; i < 14; i += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], cc, m));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i + 1], cc, m));
        const f32x2 v = {e0, e1};
        pk ^= __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
        l0 += e0;
        l1 += e1;
      }
    }
    r = l0 + l1 + (float)pk;
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
  stamp_store(out, 8, c0, c1, r0, r1);
}

// ---------------------------------------------------------------------------
// 4b. waves interleaving their own MFMAs with vector work
// ---------------------------------------------------------------------------
// Four or eight waves (one or two per SIMD), each issuing 16 v_mfma_f32_32x32x16_bf16 per K
// tile on 4 independent accumulators, with M softmax pairs per tile (per
// pair: 2 fma, 2 exp, 2 add, 1 cvt_pk_bf16, 1 xor; 8 vector instructions)
// on independent registers, scheduled as one MFMA then M/2 vector
// instructions, 16 times.  The A operand comes
//   LDSR 0: from registers;
//   LDSR 1: one 1 KiB ds_read_b128 fragment per MFMA (32 queries per wave);
//   LDSR 2: one fragment per two MFMAs against two query blocks (64 queries
//           per wave: half the LDS bytes per flop).
template <int M, int LDSR>
__global__ __launch_bounds__(512, 1) void mfma_inwave(Stamp* out, float* sink, int iters,
                                                      float seed) {
  constexpr int D = 128;
  // 32 KiB of K tiles, allocated as 96 KiB so that one work-group holds a CU
  __shared__ __attribute__((aligned(16))) __bf16 tile[64 * D * 2 * 3];
  for (int i = threadIdx.x; i < 64 * D * 2; i += blockDim.x) tile[i] = (__bf16)(seed * (float)i);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int ln = lane & 31, lh = lane >> 5;
  bf16x8 qf[8], qg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qf[ks][i] = (__bf16)(seed * (float)(lane + ks + i));
      qg[ks][i] = (__bf16)(seed * (float)(lane - ks + 2 * i));
    }
  int koff[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) koff[ks] = ln * D + (((2 * ks + lh) ^ (ln & 15)) * 8);
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = seed * (float)(threadIdx.x + 3 * i + 1);
  float l0 = 0.f, l1 = 0.f;
  unsigned pk = 0;
  const float cc = seed * 0.5f;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const __bf16* kt = tile + t * 64 * D;
      const float m = l0 * 1e-30f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        bf16x8 a0, a1;
        if constexpr (LDSR == 0) {
          a0 = qg[ks];
          a1 = qg[7 - ks];
        } else if constexpr (LDSR == 1) {
          a0 = *(const bf16x8*)(kt + koff[ks]);
          a1 = *(const bf16x8*)(kt + 32 * D + koff[ks]);
        } else {
          a0 = *(const bf16x8*)(kt + koff[ks]);
          a1 = a0;
        }
        if (ks & 1) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, LDSR == 2 ? qg[ks] : qf[ks], acc1,
                                                         0, 0, 0);
        } else {
          acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], acc2, 0, 0, 0);
          acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, LDSR == 2 ? qg[ks] : qf[ks], acc3,
                                                         0, 0, 0);
        }
      }
#pragma unroll
      for (int pr = 0; pr < M; ++pr) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[(2 * pr) & 15], cc, m));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[(2 * pr + 1) & 15], cc, m));
        const f32x2 v = {e0, e1};
        pk ^= __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
        l0 += e0;
        l1 += e1;
      }
      // schedule: the fragment reads a few ahead, then one MFMA and M / 2
      // vector instructions at a time
      if constexpr (LDSR != 0) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (LDSR == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if constexpr (LDSR == 2) {
          if (i & 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (M > 0) __builtin_amdgcn_sched_group_barrier(0x002, M / 2, 0);
      }
    }
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * blockDim.x + threadIdx.x] =
      acc0[0] + acc1[1] + acc2[2] + acc3[3] + l0 + l1 + (float)pk;
  stamp_store(out, blockDim.x >> 6, c0, c1, r0, r1);
}

// ---------------------------------------------------------------------------
// 4c. issue cost of tile loads
// ---------------------------------------------------------------------------
// Eight waves; the first `loaders` of them each issue L 1 KiB loads per
// round (64 lanes x 16 bytes, consecutive), then wait for them, then the
// work-group meets at a barrier: the attention kernels' tile-load pattern.
// KIND 0: global_load_lds_dwordx4 (to LDS through M0), 1: global_load_dwordx4
// into registers.  Per wave: cycles from the first issue to the last
// (issue) and from there to the completed wait (drain), summed over rounds.
// Each work-group reads its own 32 KiB slice per round of a buffer of
// `nbytes` (a multiple of 32 KiB), wrapping around.
template <int KIND, int L>
__global__ __launch_bounds__(512, 1) void tile_loads(Stamp* out, float* sink, const char* src,
                                                     long long nbytes, int loaders, int iters) {
  MB_RESERVE_LDS(iters);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const unsigned lds0 = (unsigned)(size_t)((MB_LDS unsigned char*)mb_pad);
  unsigned long long t_issue = 0, t_drain = 0, t_lgkm = 0;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const long long slices = nbytes / 32768;
  for (int it = 0; it < iters; ++it) {
    if (wave < loaders) {
      const long long slice = ((long long)blockIdx.x * iters + it) % slices;
      const char* base = src + slice * 32768 + (long long)wave * L * 1024;
      const unsigned m0 = __builtin_amdgcn_readfirstlane(lds0 + (unsigned)(wave * L * 1024) % 65536u);
      const unsigned long long a = __builtin_amdgcn_s_memtime();
      if constexpr (KIND == 0) {
#pragma unroll
        for (int i = 0; i < L; ++i)
          // (an SALU write of M0 needs one wait state before the LDS-DMA
          // load reads it)
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0 + i * 1024),
                       "v"((unsigned)(lane * 16 + i * 1024)), "s"(base)
                       : "memory");
      } else {
        // register loads: issued together and waited for in the same asm
        // block (so no output register is live while its load is in
        // flight); "issue" then also covers the wait
#pragma unroll
        for (int i = 0; i < L; i += 4) {
          u32x4 v0, v1, v2, v3;
          const unsigned o = (unsigned)(lane * 16 + i * 1024);
          asm volatile("global_load_dwordx4 %0, %4, %8\n\tglobal_load_dwordx4 %1, %5, %8\n\t"
                       "global_load_dwordx4 %2, %6, %8\n\tglobal_load_dwordx4 %3, %7, %8\n\t"
                       "s_waitcnt vmcnt(0)"
                       : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(v3)
                       : "v"(o), "v"(o + 1024), "v"(o + 2048), "v"(o + 3072), "s"(base)
                       : "memory");
          acc ^= v0 ^ v1 ^ v2 ^ v3;
        }
      }
      const unsigned long long b = __builtin_amdgcn_s_memtime();
      // an LDS-counter wait first: does the LDS DMA count against it?
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const unsigned long long b2 = __builtin_amdgcn_s_memtime();
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const unsigned long long c = __builtin_amdgcn_s_memtime();
      t_issue += b - a;
      t_lgkm += b2 - b;
      t_drain += c - b2;
    }
    __builtin_amdgcn_s_barrier();
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  stamp_store(out, 8, t_issue, t_drain, t_lgkm, 0);
}

// ---------------------------------------------------------------------------
// 5. one MFMA per wave, for accuracy against the exact dot products
// ---------------------------------------------------------------------------
// Problem p (one wave each): D = A B^T + C with A, B [32][K] row-major and
// C, D [32][32] fp32 row-major (D[m][n] = sum_k A[m][k] B[n][k] + C[m][n]).
// e4m3: K = 64, v_mfma_f32_32x32x64_f8f6f4 (both operands e4m3, no scaling);
// lane (l % 32, l / 32) holds bytes 32 (l / 32) .. +31 of row l % 32.
// bf16: K = 16, v_mfma_f32_32x32x16_bf16; lane holds elements 8 (l / 32) .. +7.
// Accumulator register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__global__ __launch_bounds__(64) void mfma_one_e4m3(const unsigned char* A, const unsigned char* B,
                                                    const float* C, float* D, int n) {
  const int p = blockIdx.x;
  if (p >= n) return;
  const int lane = threadIdx.x, ln = lane & 31, lh = lane >> 5;
  const i32x8 a = *(const i32x8*)(A + (long long)p * 32 * 64 + ln * 64 + 32 * lh);
  const i32x8 b = *(const i32x8*)(B + (long long)p * 32 * 64 + ln * 64 + 32 * lh);
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = C[(long long)p * 1024 + (8 * (r >> 2) + 4 * lh + (r & 3)) * 32 + ln];
  const f32x16 d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) D[(long long)p * 1024 + (8 * (r >> 2) + 4 * lh + (r & 3)) * 32 + ln] = d[r];
}

__global__ __launch_bounds__(64) void mfma_one_bf16(const __bf16* A, const __bf16* B,
                                                    const float* C, float* D, int n) {
  const int p = blockIdx.x;
  if (p >= n) return;
  const int lane = threadIdx.x, ln = lane & 31, lh = lane >> 5;
  const bf16x8 a = *(const bf16x8*)(A + (long long)p * 32 * 16 + ln * 16 + 8 * lh);
  const bf16x8 b = *(const bf16x8*)(B + (long long)p * 32 * 16 + ln * 16 + 8 * lh);
  f32x16 c;
#pragma unroll
  for (int r = 0; r < 16; ++r) c[r] = C[(long long)p * 1024 + (8 * (r >> 2) + 4 * lh + (r & 3)) * 32 + ln];
  const f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; ++r) D[(long long)p * 1024 + (8 * (r >> 2) + 4 * lh + (r & 3)) * 32 + ln] = d[r];
}

template <typename... KArgs>
static hipError_t launch(void (*kernel)(KArgs...), int grid, int block, hipStream_t stream,
                         KArgs... args) {
  void* argv[] = {static_cast<void*>(&args)..., nullptr};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), argv, 0,
                         stream);
}


// ---------------------------------------------------------------------------
// MFMA dependency: NCH accumulator chains in each wave, every MFMA reading
// its chain's previous result as SrcC, the chains issued round-robin; one or
// two waves per SIMD.  How many independent chains keep the matrix core
// busy.
// ---------------------------------------------------------------------------
template <int NCH>
__global__ __launch_bounds__(512, 1) void mfma_chain(Stamp* out, float* sink, int iters,
                                                     float seed) {
  MB_RESERVE_LDS(iters);
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(threadIdx.x + i));
    b[i] = (__bf16)(seed - (float)i);
  }
  f32x16 acc[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) acc[c] = f32x16{};
  __syncthreads();
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int c = 0; c < NCH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) r += acc[c][c];
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  stamp_store(out, blockDim.x >> 6, c0, c1, r0, r1);
  sink[blockIdx.x * blockDim.x + threadIdx.x] = r;
}

// ---------------------------------------------------------------------------
// LDS read latency: each lane follows a chain of dependent reads through an
// LDS table (the value read is the next byte address), one wave per SIMD;
// KIND 0 ds_read_b32, 1 ds_read_b128 (the next address is the first dword).
// ---------------------------------------------------------------------------
template <int KIND>
__global__ __launch_bounds__(256, 1) void lds_latency(Stamp* out, float* sink, int iters) {
  MB_RESERVE_LDS(iters);
  __shared__ __attribute__((aligned(16))) unsigned tab[4096];   // 16 KiB
  // entry i points 16 entries (64 bytes) further, wrapping: a lane's chain
  // stays inside its own 16-byte column, lanes hit different banks
  for (int i = threadIdx.x; i < 4096; i += blockDim.x) tab[i] = (unsigned)(((i + 16) & 4095) * 4);
  __syncthreads();
  unsigned addr = (unsigned)((threadIdx.x & 63) * 16);   // lane l starts at entry 4 l
  const unsigned base = (unsigned)(size_t)((MB_LDS unsigned*)tab);
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if constexpr (KIND == 0) {
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(addr) : "v"(base + addr) : "memory");
      } else {
        u32x4 v;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(base + addr) : "memory");
        addr = v[0];
      }
    }
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  stamp_store(out, blockDim.x >> 6, c0, c1, r0, r1);
  sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)addr;
}

// ---------------------------------------------------------------------------
// dQ accumulated with fp32 atomics, the traffic pattern of a causal backward
// that would add each key tile's dQ contribution into a shared fp32 buffer:
// work-group (bh, kt) of 256 threads adds a 64 x 128 fp32 tile into rows
// [64 qt, 64 qt + 64) of head bh for every 64-query tile qt >= 2 kt (the
// queries that see its 128 keys).  Wave w covers columns 32 w .. 32 w + 31;
// register r of block qb is row 32 qb + 8 (r/4) + 4 lh + r%4 (the MFMA
// accumulator layout), value (r + 1) * v.  MODE 0: agent-scope atomic add
// without return; 1: plain stores of the same addresses (the bandwidth
// reference).  Work-group L adds into head L % bh_n, so with bh_n a multiple
// of 8 all of a head's tiles run on one XCD and share its L2.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void dq_atomics(float* __restrict__ acc, int bh_n, int n, float v) {
  const int kt_n = n / 128, nq = n / 64;
  const int bh = blockIdx.x % bh_n, kt = blockIdx.x / bh_n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ln = lane & 31, lh = lane >> 5;
  (void)kt_n;
  float* base = acc + (long long)bh * n * 128 + 32 * wave + ln;
  for (int qt = 2 * kt; qt < nq; ++qt) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = qt * 64 + 32 * qb + 8 * (r >> 2) + 4 * lh + (r & 3);
        float* a = base + (long long)row * 128;
        const float x = v * (float)(r + 1);
        if constexpr (MODE == 0)
          __hip_atomic_fetch_add(a, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *a = x;
      }
  }
}
}  // namespace mb

// ---------------------------------------------------------------------------
// C entry points (device pointers; `stamps` holds grid * waves records,
// `sink` grid * threads floats).  Each returns the launch's hipError_t.
// ---------------------------------------------------------------------------
extern "C" int mb_valu_rate(int op, int grid, int waves, int iters, void* stamps, float* sink,
                            hipStream_t s) {
  if (waves < 1 || waves > 16 || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  const int blk = waves * 64;
  const float seed = 1e-3f;
  switch (op) {
    case 0: return (int)mb::launch(mb::valu_rate<0>, grid, blk, s, (mb::Stamp*)stamps, sink, iters, seed);
    case 1: return (int)mb::launch(mb::valu_rate<1>, grid, blk, s, (mb::Stamp*)stamps, sink, iters, seed);
    case 2: return (int)mb::launch(mb::valu_rate<2>, grid, blk, s, (mb::Stamp*)stamps, sink, iters, seed);
    case 3: return (int)mb::launch(mb::valu_rate<3>, grid, blk, s, (mb::Stamp*)stamps, sink, iters, seed);
    case 4: return (int)mb::launch(mb::valu_rate<4>, grid, blk, s, (mb::Stamp*)stamps, sink, iters, seed);
    case 5: return (int)mb::launch(mb::valu_rate<5>, grid, blk, s, (mb::Stamp*)stamps, sink, iters, seed);
    default: return (int)hipErrorInvalidValue;
  }
}

extern "C" int mb_mfma_pair(int acc, int grid, int mfma_waves, int valu, int iters, void* stamps,
                            float* sink, hipStream_t s) {
  if (mfma_waves < 0 || mfma_waves > 8 || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  const float seed = 1e-3f;
  if (acc == 0)
    return (int)mb::launch(mb::mfma_pair<0>, grid, 512, s, (mb::Stamp*)stamps, sink, iters,
                           mfma_waves, valu, seed);
  return (int)mb::launch(mb::mfma_pair<1>, grid, 512, s, (mb::Stamp*)stamps, sink, iters,
                         mfma_waves, valu, seed);
}

extern "C" int mb_lds_read(int kind, int grid, int waves, int iters, void* stamps, float* sink,
                           hipStream_t s) {
  if (waves < 1 || waves > 16 || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  const int blk = waves * 64;
  switch (kind) {
    case 0: return (int)mb::launch(mb::lds_read<0>, grid, blk, s, (mb::Stamp*)stamps, sink, iters);
    case 1: return (int)mb::launch(mb::lds_read<1>, grid, blk, s, (mb::Stamp*)stamps, sink, iters);
    case 2: return (int)mb::launch(mb::lds_read<2>, grid, blk, s, (mb::Stamp*)stamps, sink, iters);
    default: return (int)hipErrorInvalidValue;
  }
}

extern "C" int mb_mfma_lds(int grid, int mfma_waves, int valu, int iters, void* stamps,
                           float* sink, hipStream_t s) {
  if (mfma_waves < 0 || mfma_waves > 8 || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  return (int)mb::launch(mb::mfma_lds, grid, 512, s, (mb::Stamp*)stamps, sink, iters, mfma_waves,
                         valu, 1e-3f);
}

extern "C" int mb_mfma_inwave(int m, int ldsr, int waves, int grid, int iters, void* stamps,
                              float* sink, hipStream_t s) {
  if (grid < 1 || iters < 2 || (waves != 4 && waves != 8)) return (int)hipErrorInvalidValue;
  mb::Stamp* st = (mb::Stamp*)stamps;
#define MB_IW(M, L)                                                                          \
  if (m == M && ldsr == L)                                                                   \
    return (int)mb::launch(mb::mfma_inwave<M, L>, grid, waves * 64, s, st, sink, iters, 1e-3f);
  MB_IW(0, 0) MB_IW(4, 0) MB_IW(6, 0) MB_IW(8, 0) MB_IW(10, 0)
  MB_IW(0, 1) MB_IW(4, 1) MB_IW(6, 1) MB_IW(8, 1) MB_IW(10, 1)
  MB_IW(0, 2) MB_IW(4, 2) MB_IW(6, 2) MB_IW(8, 2) MB_IW(10, 2)
#undef MB_IW
  return (int)hipErrorInvalidValue;
}

extern "C" int mb_tile_loads(int kind, int per_wave, int loaders, int grid, int iters,
                             const void* src, long long nbytes, void* stamps, float* sink,
                             hipStream_t s) {
  if (grid < 1 || iters < 1 || loaders < 1 || loaders > 8 || nbytes < 32768 ||
      nbytes % 32768 != 0 || loaders * per_wave > 32)
    return (int)hipErrorInvalidValue;
  mb::Stamp* st = (mb::Stamp*)stamps;
  const char* p = (const char*)src;
#define MB_TL(K, Lw)                                                                           \
  if (kind == K && per_wave == Lw)                                                             \
    return (int)mb::launch(mb::tile_loads<K, Lw>, grid, 512, s, st, sink, p, nbytes, loaders, iters);
  MB_TL(0, 2) MB_TL(0, 4) MB_TL(0, 8) MB_TL(1, 4) MB_TL(1, 8)
#undef MB_TL
  return (int)hipErrorInvalidValue;
}

extern "C" int mb_mfma_one(int dtype, const void* A, const void* B, const float* C, float* D,
                           int n, hipStream_t s) {
  if (n < 1) return (int)hipErrorInvalidValue;
  if (dtype == 0)
    return (int)mb::launch(mb::mfma_one_e4m3, n, 64, s, (const unsigned char*)A,
                           (const unsigned char*)B, C, D, n);
  return (int)mb::launch(mb::mfma_one_bf16, n, 64, s, (const __bf16*)A, (const __bf16*)B, C, D, n);
}

extern "C" int mb_mfma_chain(int nch, int waves, int grid, int iters, void* stamps, float* sink,
                             hipStream_t s) {
  if (grid < 1 || iters < 1 || (waves != 4 && waves != 8)) return (int)hipErrorInvalidValue;
  mb::Stamp* st = (mb::Stamp*)stamps;
  const int blk = waves * 64;
  switch (nch) {
    case 1: return (int)mb::launch(mb::mfma_chain<1>, grid, blk, s, st, sink, iters, 1e-3f);
    case 2: return (int)mb::launch(mb::mfma_chain<2>, grid, blk, s, st, sink, iters, 1e-3f);
    case 3: return (int)mb::launch(mb::mfma_chain<3>, grid, blk, s, st, sink, iters, 1e-3f);
    case 4: return (int)mb::launch(mb::mfma_chain<4>, grid, blk, s, st, sink, iters, 1e-3f);
    default: return (int)hipErrorInvalidValue;
  }
}

extern "C" int mb_lds_latency(int kind, int grid, int iters, void* stamps, float* sink,
                              hipStream_t s) {
  if (grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  mb::Stamp* st = (mb::Stamp*)stamps;
  if (kind == 0) return (int)mb::launch(mb::lds_latency<0>, grid, 256, s, st, sink, iters);
  if (kind == 1) return (int)mb::launch(mb::lds_latency<1>, grid, 256, s, st, sink, iters);
  return (int)hipErrorInvalidValue;
}

// acc: bh_n * n * 128 floats on the device; n a multiple of 128
extern "C" int mb_dq_atomics(int mode, int bh_n, int n, float* acc, float v, hipStream_t s) {
  if (bh_n < 1 || n < 128 || n % 128 != 0 || acc == nullptr) return (int)hipErrorInvalidValue;
  const int grid = bh_n * (n / 128);
  if (mode == 0) return (int)mb::launch(mb::dq_atomics<0>, grid, 256, s, acc, bh_n, n, v);
  if (mode == 1) return (int)mb::launch(mb::dq_atomics<1>, grid, 256, s, acc, bh_n, n, v);
  return (int)hipErrorInvalidValue;
}
