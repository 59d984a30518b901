// Device helpers and host launch checks shared by the kernel files of libsq
// (gfx950 / MI355X).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstring>
#include <limits>
#include <string>
#include <type_traits>
#include <vector>

#include "internal.h"

namespace sq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float((uint32_t)u << 16);
}

// float -> bfloat16 bits, round to nearest even (finite inputs)
__host__ __device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t half_bits_rne(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float half_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// Uniform table reads go through the constant address space so that they
// become scalar loads: the compiler can then neither confuse them with the
// kernel's own global stores nor make them wait for those stores.
#define SQ_CONST __attribute__((address_space(4)))
template <typename T>
__device__ __forceinline__ const SQ_CONST T *cptr(const void *p) {
  return (const SQ_CONST T *)(uintptr_t)p;
}
__device__ __forceinline__ DevCoord load_coord(const SQ_CONST DevCoord *p) {
  DevCoord r;
  r.bit_off = p->bit_off;
  r.width = p->width;
  r.thr_base = p->thr_base;
  r.cent_base = p->cent_base;
  return r;
}

// Wait for this wave's LDS operations and keep the compiler from moving LDS
// accesses across this point (cross-lane exchange within one wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n (the counter field is an immediate)
__device__ __forceinline__ void wait_vmcnt(int n) {
  switch (n) {
#define SQ_VMW(k) \
  case k: __builtin_amdgcn_s_waitcnt(0x0F70 | ((k) & 15) | (((k) >> 4) << 14)); break;
#define SQ_VMW8(k) SQ_VMW(k) SQ_VMW(k + 1) SQ_VMW(k + 2) SQ_VMW(k + 3) SQ_VMW(k + 4) SQ_VMW(k + 5) SQ_VMW(k + 6) SQ_VMW(k + 7)
    SQ_VMW8(0) SQ_VMW8(8) SQ_VMW8(16) SQ_VMW8(24) SQ_VMW8(32) SQ_VMW8(40) SQ_VMW8(48) SQ_VMW8(56)
#undef SQ_VMW8
#undef SQ_VMW
    default: __builtin_amdgcn_s_waitcnt(0xCF7F); break;  // vmcnt(63): waits for more, never less
  }
}

// workgroup barrier without the memory fence of __syncthreads (the producer
// must not wait for its later loads); LDS writes of the wave are complete.
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct-to-LDS loads (global_load_lds_dword / _dwordx4): lane l's 4 (16)
// bytes land at LDS address lds + 4l (16l).  Written as asm so that the
// compiler does not treat every later LDS read of the workgroup as a possible
// reader of these writes (it would wait for all vector memory there); the
// loads are ordered explicitly by wait_vmcnt and step_barrier.  They have no
// register results.
// Address = wave-uniform base (scalar pair) + per-lane byte offset.
__device__ __forceinline__ void lds_dma16(const void *base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void *base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}
// a wave-uniform value kept in a vector register (it is combined with
// another uniform operand in one VOP3 instruction, which takes one scalar)
__device__ __forceinline__ uint32_t to_vgpr(uint32_t x) {
  uint32_t v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(x));
  return v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a),
                                                __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_pair(uint16_t x) { return (uint32_t)x | ((uint32_t)x << 16); }

// Maximum over the 64 lanes (returned in every lane), on order-preserving
// integer keys of the floats (sign-magnitude to two's complement): rotations
// within each row of 16 (DPP), then the four row results.  A positive NaN
// wins and a negative NaN loses; either way its token's weight is NaN.
__device__ __forceinline__ float wave_max(float v) {
  int k = __float_as_int(v);
  k ^= (k >> 31) & 0x7FFFFFFF;
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x128, 0xF, 0xF, true));  // (row rotations: every lane valid)
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x124, 0xF, 0xF, true));
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x122, 0xF, 0xF, true));
  k = max(k, __builtin_amdgcn_mov_dpp(k, 0x121, 0xF, 0xF, true));
  int m = max(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)),
              max(__builtin_amdgcn_readlane(k, 32), __builtin_amdgcn_readlane(k, 48)));
  m ^= (m >> 31) & 0x7FFFFFFF;
  return __int_as_float(m);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// (bf16(x), bf16(x)) packed, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16_pair_rne(float x) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x, x}, bf16x2_t));
}

// ------------------------------------------------------------------ host checks

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static inline sq_status hip_fail(const char *what, hipError_t e) {
  return fail(SQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

static inline int device_lds_limit() {
  int dev = 0, v = 65536;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  return v;
}

static inline sq_status check_handle(const sq_calib *c, const char *fn) {
  if (!c) return fail(SQ_ERR_ARG, std::string(fn) + ": handle is NULL");
  if (!c->dev_blob) return fail(SQ_ERR_STATE, std::string(fn) + ": calibration not uploaded (call sq_calib_upload)");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(fn, e);
  if (dev != c->device)
    return fail(SQ_ERR_STATE, std::string(fn) + ": calibration was uploaded to another device");
  return SQ_OK;
}

// calibration heads used: first_head + b*cbs + h for b < batch, h < n_heads
static inline sq_status check_heads(const sq_calib *c, int first_head, int n_heads, int batch, int cbs,
                             const char *fn) {
  const int64_t nh = (int64_t)c->heads.size();
  if (n_heads <= 0 || batch < 0 || cbs < 0 || first_head < 0)
    return fail(SQ_ERR_ARG, std::string(fn) + ": bad head range (need n_heads > 0, batch, cbs, first_head >= 0)");
  const int64_t last = (int64_t)first_head + (int64_t)std::max(0, batch - 1) * cbs + n_heads - 1;
  if (last >= nh) return fail(SQ_ERR_ARG, std::string(fn) + ": calibration head index out of range");
  const int d = c->heads[first_head].d;
  for (int64_t k = first_head; k <= last; ++k)
    if (c->heads[k].d != d) return fail(SQ_ERR_ARG, std::string(fn) + ": heads of different head_dim");
  return SQ_OK;
}

static inline sq_status check_slots(const sq_calib *c, int64_t n_tokens, int n_heads, int batch, int64_t ps_b,
                             int64_t ps_h, const char *fn) {
  const int64_t need = ((n_tokens + 63) / 64) * 64 * (int64_t)c->W_max;
  if (ps_h < need) return fail(SQ_ERR_ARG, std::string(fn) + ": ps_head smaller than sq_packed_head_words");
  if (batch > 1 && ps_b < ps_h * n_heads) return fail(SQ_ERR_ARG, std::string(fn) + ": ps_batch overlaps head slots");
  return SQ_OK;
}

// Paged packed cache.  Tile `tile` (64 tokens) of (batch row b, head h of
// the call) lives in physical block table[b * tstride + tile / bt], at word
// (block * nh + h) * block_words + (tile % bt) * W * 64 of the pool; a block
// holds bt tiles of each of the call's nh heads.  table == nullptr: the
// contiguous slots of the unpaged calls.
struct PageArgs {
  const int32_t *table;
  int64_t tstride, block_words;
  int32_t bt, nh, n_blocks, pad;
};

// Word 0 of a tile for reads (wave-uniform): contiguous slot + tile * W * 64,
// or the tile in its block; a block id outside [0, n_blocks) is clamped, so a
// bad table entry can never address memory outside the pool.
__device__ __forceinline__ const uint32_t *page_tile(const PageArgs &pg, const uint32_t *slot_or_pool, int b,
                                                     int h, int64_t tile, int W) {
  if (!pg.table) return slot_or_pool + tile * W * 64;
  // (tiles of one row stay below 2^31: the host limits tokens to 2^36)
  const uint32_t t32 = (uint32_t)tile, lb = t32 / (uint32_t)pg.bt, tb = t32 - lb * (uint32_t)pg.bt;
  int64_t blk = pg.table[(int64_t)b * pg.tstride + lb];
  blk = blk < 0 ? 0 : blk >= pg.n_blocks ? pg.n_blocks - 1 : blk;
  return slot_or_pool + (blk * pg.nh + h) * pg.block_words + (int64_t)tb * W * 64;
}

// Word 0 of destination token dtok for writes (per lane); nullptr for a
// block id outside [0, n_blocks) (the words are dropped).
__device__ __forceinline__ uint32_t *page_token(const PageArgs &pg, uint32_t *slot_or_pool, int b, int h,
                                                int64_t dtok, int W) {
  const int64_t tile = dtok >> 6;
  if (!pg.table) return slot_or_pool + tile * W * 64 + (dtok & 63);
  const uint32_t t32 = (uint32_t)tile, lb = t32 / (uint32_t)pg.bt, tb = t32 - lb * (uint32_t)pg.bt;
  const int64_t blk = pg.table[(int64_t)b * pg.tstride + lb];
  if (blk < 0 || blk >= pg.n_blocks) return nullptr;
  return slot_or_pool + (blk * pg.nh + h) * pg.block_words + (int64_t)tb * W * 64 + (dtok & 63);
}

// Word 0 of destination token token0 + 64 tile + lane for writes from one
// source tile (wave-uniform tile; token0 may be unaligned, so the wave's
// lanes fall into destination tiles d0 = token0 / 64 + tile and d0 + 1):
// the two blocks are looked up once per wave through the scalar cache, the
// second only when some lane lands in it (last_dtile: the call's last
// destination tile).  nullptr for a block id outside [0, n_blocks).
__device__ __forceinline__ uint32_t *page_token_tile(const PageArgs &pg, uint32_t *pool, int b, int h,
                                                     int64_t token0, int64_t tile, int lane, int64_t last_dtile,
                                                     int W) {
  const SQ_CONST int32_t *row = (const SQ_CONST int32_t *)(pg.table + (int64_t)b * pg.tstride);
  const uint32_t d0 = (uint32_t)((token0 >> 6) + tile);  // tiles of one row stay below 2^31
  const uint32_t lb0 = d0 / (uint32_t)pg.bt, tb0 = d0 - lb0 * (uint32_t)pg.bt;
  const uint32_t d1 = d0 + 1u, lb1 = tb0 + 1u == (uint32_t)pg.bt ? lb0 + 1u : lb0;
  const uint32_t tb1 = tb0 + 1u == (uint32_t)pg.bt ? 0u : tb0 + 1u;
  const int32_t blk0 = row[lb0];
  const int32_t blk1 = (int64_t)d1 <= last_dtile ? row[lb1] : -1;
  const bool hi = (int)(token0 & 63) + lane >= 64;
  const int32_t blk = hi ? blk1 : blk0;
  if (blk < 0 || blk >= pg.n_blocks) return nullptr;
  const uint32_t tb = hi ? tb1 : tb0;
  return pool + ((int64_t)blk * pg.nh + h) * pg.block_words + (int64_t)tb * W * 64 + ((token0 + lane) & 63);
}

// Host checks of a paged cache description for a call that touches tokens
// [0, n_tokens) of each batch row; fills the kernels' PageArgs.
static inline sq_status check_paged(const sq_calib *c, const sq_paged *pg, int64_t n_tokens, int n_heads,
                                    const char *fn, PageArgs &out) {
  const std::string f(fn);
  if (!pg || !pg->block_table) return fail(SQ_ERR_ARG, f + ": paged cache without a block table");
  if (pg->block_tiles < 1 || pg->n_blocks < 1) return fail(SQ_ERR_ARG, f + ": block_tiles and n_blocks must be >= 1");
  const int64_t tiles = (n_tokens + 63) / 64;
  const int64_t blocks = (tiles + pg->block_tiles - 1) / pg->block_tiles;
  if (pg->table_stride < blocks) return fail(SQ_ERR_ARG, f + ": table_stride below the logical blocks of the call");
  out = PageArgs{};
  out.table = pg->block_table;
  out.tstride = pg->table_stride;
  out.block_words = (int64_t)pg->block_tiles * 64 * c->W_max;
  out.bt = pg->block_tiles;
  out.nh = n_heads;
  out.n_blocks = pg->n_blocks;
  return SQ_OK;
}

static inline sq_status launched(const char *fn) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(fn, e);
  clear_error();
  return SQ_OK;
}

static inline int device_cu_count() {
  int dev = 0, v = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  return v;
}

// Summary of sq_scores' launch plan (scores.hip), for sq_plan_decode.
sq_status score_plan_summary(const sq_calib *kc, int first_head, int calib_batch_stride, int batch,
                             int n_q_heads, int n_kv_heads, int64_t n_tokens, int *passes, int *max_quads,
                             int *wave_groups);

}  // namespace sq
