// q2_unit.h -- the integer dot of one 64-weight Q2 unit against int8
// activations, shared by the GEMV kernels.
//
// What is computed (qxmx qxmx_gpu.cpp page, gemv_dpas8): the corrected dot
//     sum_{i in unit} code_i * xq_i - suma,   suma = sum_{i in unit} xq_i,
// which equals sum (code_i - 1) * xq_i exactly.
//
// Code layout (fixed by the repack): a unit is four 32-bit words; field a
// (bits 2a..2a+1 of each byte) of word j holds the codes of activation word
// 4j + a, so (word >> 2a) & 0x03030303 lines up with that word.
//
// Instruction count: a field need not sit at bit 0 to be a dot4 operand.
// Field 1 masked in place (word & 0x0C0C0C0C) is 4 x code, still a
// non-negative int8, so its dot4 is exactly 4x the field's dot; fields 2 and
// 3 are the same after one shift by 4.  Fields 0 and 2 accumulate in p1 and
// fields 1 and 3 in p4, and p4 / 4 (an exact shift: every term is a
// multiple of 4) joins them at the end: per word one shift and four masks
// instead of three shifts and four masks, and the integer result is the
// same.  |p4| <= 4 * 32 * 3 * 128, far inside int32.
#pragma once

namespace qg {

typedef int q2_i32x4 __attribute__((ext_vector_type(4)));

__device__ inline void q2_word_dot(unsigned w, int x0, int x1, int x2, int x3, int &p1, int &p4) {
  const unsigned h = w >> 4;
  p1 = __builtin_amdgcn_sdot4((int)(w & 0x03030303u), x0, p1, false);
  p4 = __builtin_amdgcn_sdot4((int)(w & 0x0C0C0C0Cu), x1, p4, false);
  p1 = __builtin_amdgcn_sdot4((int)(h & 0x03030303u), x2, p1, false);
  p4 = __builtin_amdgcn_sdot4((int)(h & 0x0C0C0C0Cu), x3, p4, false);
}

// Corrected dot of one unit: codes c (four words), activation words
// x0..x3 (four int8 each, natural order), suma sa.
__device__ inline int q2_unit_dot(const q2_i32x4 c, const q2_i32x4 x0, const q2_i32x4 x1, const q2_i32x4 x2,
                                  const q2_i32x4 x3, int sa) {
  int p1 = 0, p4 = 0;
  q2_word_dot((unsigned)c.x, x0.x, x0.y, x0.z, x0.w, p1, p4);
  q2_word_dot((unsigned)c.y, x1.x, x1.y, x1.z, x1.w, p1, p4);
  q2_word_dot((unsigned)c.z, x2.x, x2.y, x2.z, x2.w, p1, p4);
  q2_word_dot((unsigned)c.w, x3.x, x3.y, x3.z, x3.w, p1, p4);
  return p1 + (p4 >> 2) - sa;
}

}  // namespace qg
