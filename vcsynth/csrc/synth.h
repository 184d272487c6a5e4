/* GPU fill entry points of the seeded input generator (see vcsynth/rng.py for the definition).
 * dst is device memory; element e of the dense row-major tensor `shape` gets the draw at logical
 * index lbase + sum_k coord_k * lstride[k].  Return 0 on success, -1 bad argument, -3 HIP error. */
#ifndef VCSYNTH_H
#define VCSYNTH_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
/* bf16 normal variates: values has ntab + 1 entries, thresholds ntab (device arrays). */
int vcs_fill_normal_bf16(void* dst, int ndim, const int64_t* shape, const int64_t* lstride,
                         int64_t lbase, uint64_t seed, uint32_t stream_id, const uint32_t* thresholds,
                         const uint16_t* values, int ntab, void* stream);
/* raw upper 32 bits of each draw */
int vcs_fill_u32(void* dst, int ndim, const int64_t* shape, const int64_t* lstride, int64_t lbase,
                 uint64_t seed, uint32_t stream_id, void* stream);
#ifdef __cplusplus
}
#endif
#endif
