"""CPU oracle for the Flash-Cache step: test infrastructure, never product code."""
