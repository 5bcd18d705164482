// Host-side helpers shared by the host calls (rotation from prefill vectors,
// segment strategy generation).
#pragma once
#include <stdint.h>

#include <vector>

#include "../../include/mkv.h"

namespace mkv {

// element i of a host array in the storage dtype (f32 values or bf16 bit patterns), as binary64
double host_elem(const void *x, int32_t dtype, int64_t i);

// Eigenvectors of the symmetric d x d matrix G (row-major, both triangles;
// overwritten): Householder tridiagonalisation and the implicit symmetric QR
// iteration, rows ordered by descending eigenvalue, the largest-magnitude
// entry of each row made positive (ties to the lower index). R_out [d][d]
// float32; sigma_out [d] (nullable) = sqrt(max(eigenvalue, 0)).
mkv_status rotation_from_gram(std::vector<double> &G, int d, float *R_out, double *sigma_out);

}  // namespace mkv
