// Validation helpers shared by check.cpp and the kernels' host code (not part
// of the C ABI).  No HIP types: check.cpp builds with a plain host compiler.
#ifndef SATTN_CHECK_H
#define SATTN_CHECK_H

// The validation of sattn_bwd_key_noalloc: sattn_bwd_key_check's rules with
// the workspace replaced by the library's static region of `scratch_bytes`
// bytes (SATTN_ERR_SCRATCH when the problem needs more).
int sattn_bwd_key_noalloc_check(const void* Q, const void* K, const void* Vt, const void* dO,
                                const float* L, const float* D, const float* dK,
                                const float* dVt, float c, float s, int T, int Hq, int Hkv,
                                unsigned long long scratch_bytes);

#endif  // SATTN_CHECK_H
