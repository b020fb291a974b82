// Device-side building blocks for the NVFP4 weight pass on gfx950 (CDNA4).
//
// Element formats ("NVFP4 group-16", dgx-spark-qwen38 README, "The seven
// targets"): E2M1 codes two per byte (element 2j = low nibble of byte j),
// one E4M3 block scale per 16 K-elements, an fp32 tensor scale.
//
// Decoding uses the gfx950 conversion instructions:
//   v_cvt_scalef32_pk_{f32,bf16}_fp4  two E2M1 codes of one byte -> two
//     values, low nibble first.  Its scale operand contributes only its
//     exponent, so it is always passed 1.0 here and the E4M3 scale (which
//     has a mantissa) is applied with an ordinary multiply.
//   v_cvt_scalef32_pk_f32_fp8  two E4M3 bytes -> two fp32, exact for every
//     code including subnormals.
// Every product x * s * e is exact in fp32 (8 + 4 + 2 significant bits) and
// s * e is exact in bf16 (6 bits), so the only rounding is the fp32
// accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vg {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---- loads -------------------------------------------------------------
// Every buffer the kernels touch is global device memory.  Pointers read
// from a device-side job table carry no address space, and generic (FLAT)
// accesses would count against the LDS/scalar wait counter too, so every
// access goes through an explicit global (address space 1) pointer.
#define VG_GLOBAL __attribute__((address_space(1)))

// Weight bytes are read exactly once per pass: nontemporal (streaming) hint.
__device__ __forceinline__ u32x4 ld_stream(const u32x4* p) {
  return __builtin_nontemporal_load((const VG_GLOBAL u32x4*)p);
}
__device__ __forceinline__ unsigned short ld_stream(const unsigned short* p) {
  return __builtin_nontemporal_load((const VG_GLOBAL unsigned short*)p);
}
__device__ __forceinline__ unsigned ld_stream(const unsigned* p) {
  return __builtin_nontemporal_load((const VG_GLOBAL unsigned*)p);
}
__device__ __forceinline__ unsigned char ld_stream(const unsigned char* p) {
  return __builtin_nontemporal_load((const VG_GLOBAL unsigned char*)p);
}
// Activations are small and re-read by many workgroups: ordinary cached loads.
__device__ __forceinline__ u32x4 ld_act(const u32x4* p) { return *(const VG_GLOBAL u32x4*)p; }

// ---- decoding ----------------------------------------------------------
// Two E4M3 scale bytes (low 16 bits of w) -> two fp32 values.
__device__ __forceinline__ f32x2 e4m3x2_lo(unsigned w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
}
__device__ __forceinline__ f32x2 e4m3x2_hi(unsigned w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
}

// Byte `sel` of a code dword -> bf16 pair (element 2*sel, 2*sel+1), unscaled.
template <int sel>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(unsigned w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, sel);
}
// Byte `sel` of a code dword -> fp32 pair, unscaled.
template <int sel>
__device__ __forceinline__ f32x2 e2m1x2_f32(unsigned w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, sel);
}

// Two fp32 values that bf16 holds exactly (a = s * e has at most 6
// significant bits, so the low 16 bits of its fp32 form are zero) as a
// bf16 pair: their high halves, gathered by one byte permute (v_perm_b32
// runs at twice the rate of the fp32-to-bf16 conversion).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  return __builtin_amdgcn_perm(__builtin_bit_cast(unsigned, b), __builtin_bit_cast(unsigned, a), 0x07060302u);
}

// One code dword (8 elements of one 16-block) times its block scale s, as
// the bf16x8 B-operand of an MFMA: element order is the K order.
__device__ __forceinline__ bf16x8 dequant8_bf16(unsigned w, float s) {
  f32x2 p0 = e2m1x2_f32<0>(w), p1 = e2m1x2_f32<1>(w), p2 = e2m1x2_f32<2>(w), p3 = e2m1x2_f32<3>(w);
  u32x4 r;
  r[0] = pack_bf16x2(p0[0] * s, p0[1] * s);
  r[1] = pack_bf16x2(p1[0] * s, p1[1] * s);
  r[2] = pack_bf16x2(p2[0] * s, p2[1] * s);
  r[3] = pack_bf16x2(p3[0] * s, p3[1] * s);
  return __builtin_bit_cast(bf16x8, r);
}

// A dword holding two bf16 values as a bf16x2 operand.  The dword is taken
// by value on purpose: __builtin_bit_cast applied directly to an element of
// an ext_vector (x[1]) reinterprets the vector's first dword instead.
__device__ __forceinline__ bf16x2 as_bf16x2(unsigned v) { return __builtin_bit_cast(bf16x2, v); }

// sum_{j<8} x_j * e_j for one code dword against four dwords of bf16 pairs.
__device__ __forceinline__ float dot8(unsigned w, u32x4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<0>(w), as_bf16x2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<1>(w), as_bf16x2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<2>(w), as_bf16x2(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_bf16<3>(w), as_bf16x2(x.w), acc, false);
  return acc;
}

// FP8 (E4M3) weights: bytes 2*hi and 2*hi+1 of a dword -> two bf16, exact
// (E4M3 values have 4 significant bits and exponents within bf16's range).
template <bool hi>
__device__ __forceinline__ bf16x2 e4m3x2_bf16(unsigned w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, hi);
}
// A buffer descriptor over `bytes` bytes at `base` (raw, stride 0): loads
// at offsets past `bytes` return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// rsrc for a base and range that are wave-uniform in fact but that the
// compiler may not prove uniform: both go through readfirstlane, so the
// descriptor lives in scalar registers (a descriptor in vector registers
// makes the compiler wrap every load in a loop over its distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_uniform(const void* base, unsigned bytes) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  // readfirstlane returns a signed int: widen through unsigned, or a low
  // word with bit 31 set would sign-extend into the high word
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const unsigned long long u = ((unsigned long long)hi << 32) | (unsigned long long)lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0,
                                           (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// The same buffer descriptor as four scalar words, for dma16.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, unsigned bytes) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)b);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32)) & 0xFFFFu;  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

// LDS address (byte offset) of a location in LDS.
template <class T>
__device__ __forceinline__ unsigned lds_addr(T* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) T*)p;
}

// One 1-KB global-to-LDS copy: lane i's 16 bytes at byte `voff` of buffer
// `rs` land at LDS byte lds + 16 * i.  An offset past the buffer's range
// reads nothing from memory, but the lane still writes its 16 LDS bytes,
// so every lane's destination must lie inside the area being filled.
// Written as assembly so that the compiler does not track it: it would
// otherwise wait for every LDS copy in flight before any LDS read of this
// wave (including the copies made ahead of time).  Completion is awaited
// explicitly (vmcnt) by the caller.  The compiler emits no other LDS copy,
// so it keeps nothing in M0 across this.  `lds` must be wave-uniform; it is
// moved to a scalar register here (the "s" constraint alone does not make
// the compiler move a value that lives in a vector register).
__device__ __forceinline__ void dma16(u32x4 rs, unsigned voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "s"(m)
               : "memory", "m0");
}
// dma16 at device scope (sc1): each dword is read as an agent-scope relaxed
// atomic load reads it (past the XCD's non-coherent L2), so data that
// another workgroup wrote and acknowledged before a counter this wave has
// seen is read fresh without an acquire fence.
__device__ __forceinline__ void dma16_agent(u32x4 rs, unsigned voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen sc1 lds" ::"v"(voff), "s"(rs), "s"(m)
               : "memory", "m0");
}

// s_waitcnt immediate for vmcnt(n) alone (gfx9 encoding: vmcnt bits 3:0
// and 15:14; expcnt 7 and lgkmcnt 15 = no wait on those).
constexpr unsigned vmcnt_imm(unsigned n) { return (n & 15u) | ((n >> 4) << 14) | 0x0F70u; }

// Eight E4M3 weights (two dwords, element order = byte order) dotted with
// eight bf16 activations (one 16-byte piece), accumulated onto acc.
__device__ __forceinline__ float fp8_dot8(unsigned w0, unsigned w1, u32x4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_bf16<false>(w0), as_bf16x2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_bf16<true>(w0), as_bf16x2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_bf16<false>(w1), as_bf16x2(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(e4m3x2_bf16<true>(w1), as_bf16x2(x.w), acc, false);
  return acc;
}
// Eight E4M3 weights as the bf16x8 operand of a bf16 MFMA.
__device__ __forceinline__ bf16x8 fp8x8_bf16(unsigned w0, unsigned w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(unsigned, e4m3x2_bf16<false>(w0));
  r[1] = __builtin_bit_cast(unsigned, e4m3x2_bf16<true>(w0));
  r[2] = __builtin_bit_cast(unsigned, e4m3x2_bf16<false>(w1));
  r[3] = __builtin_bit_cast(unsigned, e4m3x2_bf16<true>(w1));
  return __builtin_bit_cast(bf16x8, r);
}

// One 16-element block: codes (2 dwords), x (4 dwords-of-pairs x 2), scale.
__device__ __forceinline__ float block16(unsigned c0, unsigned c1, u32x4 xa, u32x4 xb, float s,
                                         float acc) {
  float p = dot8(c0, xa, 0.0f);
  p = dot8(c1, xb, p);
  return __builtin_fmaf(s, p, acc);
}

// ---- reductions ----------------------------------------------------------
// Sum over each half-wave (lanes 0-31, 32-63) with DPP moves only (no LDS
// permute): quad swaps, row rotations by 4 and 8 (every lane of a 16-lane
// row then holds the row sum), then row_bcast15 adds row 0's sum into row
// 1 and row 2's into row 3.  The half-wave sums are valid in lanes 16-31
// and 48-63.  A fixed pattern, so the result is bitwise repeatable.
__device__ __forceinline__ float half_wave_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  return v;
}

template <int width>
__device__ __forceinline__ float sum_lanes(float v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// ---- argmax keys -----------------------------------------------------------
// A (logit, index) pair packed so that unsigned 64-bit max picks the larger
// logit, and among equal logits the LOWER index.  -0 is canonicalised to +0
// so that the two zeros compare equal, as they do as numbers.
__device__ __forceinline__ unsigned long long argmax_key(float v, unsigned idx) {
  v = v + 0.0f;  // -0 + 0 = +0 under round-to-nearest
  unsigned u = __float_as_uint(v);
  unsigned ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ unsigned key_index(unsigned long long key) {
  return 0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull);
}

// Better = larger logit, then lower index.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

}  // namespace vg
