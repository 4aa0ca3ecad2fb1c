/*
 * lrs_oracle.c -- plain sequential CPU reference for the linear-recurrence
 * scans (first-order FMA and gated scans and their reverse (gradient) passes,
 * decay-separable outer-product state scan, delta-rule state scan with and
 * without a per-key decay, and an explicit second form of each delta rule).
 *
 * TEST INFRASTRUCTURE ONLY.  This file, its Python wrapper and everything
 * else under oracle/ exist to check the GPU library.  Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load or
 * call it.  It shares no source, header, table or helper with the GPU path,
 * and the GPU path never calls it.
 *
 * Sources, cited by short name:
 *   [SunnyNet log]   "SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的 C 推理运行时",
 *                    developer.aliyun.com/article/1773847
 *   [vs llama.cpp]   "我拿同一份权重和 llama.cpp 正面比了一场：我手写的 C 内核，慢了 1.1–1.7 倍",
 *                    developer.aliyun.com/article/1775078
 *
 * Build (no fast-math, no contraction, so each statement rounds as written):
 *   gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC \
 *       lrs_oracle.c -o liblrs_oracle.so -lm
 *
 * Each (b, n) channel or (b, h) head is computed by exactly one thread with
 * the same arithmetic, so results are bit-identical for any thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define ORC_NBLK 256 /* channels advanced together per work item (memory order only) */

#define REAL double
#define SFX _f64
#define ORC_EXP exp
#include "lrs_oracle_impl.h"
#undef REAL
#undef SFX
#undef ORC_EXP

#define REAL float
#define SFX _f32
#define ORC_EXP expf
#include "lrs_oracle_impl.h"
#undef REAL
#undef SFX
#undef ORC_EXP

/* Version of this oracle's arithmetic; bumped whenever a formula changes. */
int orc_version(void) { return 4; }
