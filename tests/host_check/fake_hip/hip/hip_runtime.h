// Minimal host-only stand-in for the HIP runtime header, for building the C
// ABI's host code (capi.cpp) with g++ and the address / undefined-behaviour
// sanitizers on a machine without a GPU.  Only what capi.cpp uses.
#pragma once
#include <cstddef>
#include <cstdint>

typedef int hipError_t;
constexpr hipError_t hipSuccess = 0;
typedef struct ihipStream_t *hipStream_t;
typedef struct ihipEvent_t *hipEvent_t;
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 1 };

hipError_t hipGetDevice(int *device);
hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t attr, int device);
hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream);
